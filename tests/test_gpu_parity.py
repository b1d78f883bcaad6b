"""GPU parity of the HIP path (through the C interface) against the fp64 oracle.

Scores: scaled error <= 2e-3 (see tests/_parity.py). Select: bit-exact against the top-B of the
GPU's own scores, and equal to the oracle's kept set except for keys inside the tolerance band
around the B-th score. Compaction: byte-exact; rows past the kept count untouched.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle as O
from synthgen import pack_units, workload
from tests._parity import SPLIT_ROWS, TOL, candidate_profile, check_unit, gen_workers, oracle_unit, run_gpu, score_error, widen

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def margin(config, err, mism, units):
    """One line of the parity-margin record: the largest scaled score error against the oracle
    and the keys whose kept status differs from the oracle's (each inside the tolerance band)."""
    say(f"[margin] {config} | {err:.3g} | {mism} | {units}")


def test_c1_full():
    wl = workload("c1")
    say("case c1: 1 x 4096 fp32 keys, B=256")
    P = pack_units(wl)
    out = run_gpu(P, wl, wl.budget)
    err, mism = check_unit(P, 0, wl, out, wl.budget, label="c1")
    say(f"c1 score err {err:.3g}, kept mismatches in band {mism}")
    margin("C1 (1 x 4096 fp32, B=256)", err, mism, 1)
    assert out["ws_after"]  # workspace back at rest


def test_c2_full():
    wl = workload("c2")
    say("case c2: 8 x 32768 bf16 keys, B=2048")
    P = pack_units(wl, workers=gen_workers())
    out = run_gpu(P, wl, wl.budget)
    worst, total = 0.0, 0
    for i in range(wl.n_units):
        err, mism = check_unit(P, i, wl, out, wl.budget, label="c2")
        worst, total = max(worst, err), total + mism
    say(f"c2 worst score err {worst:.3g}, kept mismatches in band {total}")
    margin("C2 (8 x 32768 bf16, B=2048)", worst, total, wl.n_units)
    assert out["ws_after"]
    # the three separate calls, the standalone select (its own histogram) and the split select
    # path (candidate, resolve, emit kernels) give the same bits
    for path, mr in [("calls", None), ("standalone", None), ("fused", SPLIT_ROWS), ("standalone", SPLIT_ROWS)]:
        out2 = run_gpu(P, wl, wl.budget, path=path, max_rows=mr)
        for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
            assert np.array_equal(out2[k], out[k]), (path, mr, k)
        assert out2["ws_after"], (path, mr)
    # deterministic: a second pass is bitwise identical
    out3 = run_gpu(P, wl, wl.budget)
    for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
        assert np.array_equal(out3[k], out[k]), k


def test_passes_on_two_streams():
    """Passes issued over two streams, copy c always on stream c % 2 with its own workspace and
    outputs, as a loop compressing layer after layer may issue them: every copy ends bitwise equal
    to the same pass run alone on one stream (no state shared between calls)."""
    import rotary_frequency_key_amd as tri
    from tests._parity import keys_to_device

    wl = workload("c2")
    P = pack_units(wl, [0, 1, 2], [32768, 20000, 700])
    U, B, dev = 3, wl.budget, torch.device("cuda:0")
    max_rows = int(np.diff(P["row_off"]).max())
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, np.array([1 << j for j in range(17)]), P["centers"][:U])
    say("case two streams, 4 copies")

    def copy_plan():
        c = dict(K=keys_to_device(P["keys"], wl.dtype, dev), V=keys_to_device(P["values"], wl.dtype, dev),
                 pos=torch.from_numpy(P["pos"]).to(dev), row_off=torch.from_numpy(P["row_off"]).to(dev),
                 t=torch.from_numpy(P["t"]).to(dev), mu=torch.from_numpy(mu).to(dev))
        outs = dict(kept_idx=torch.full((U, B), -7, dtype=torch.int32, device=dev),
                    kept_cnt=torch.empty(U, dtype=torch.int32, device=dev),
                    K_out=torch.zeros((U, B, wl.d), dtype=torch.bfloat16, device=dev),
                    V_out=torch.zeros((U, B, wl.d), dtype=torch.bfloat16, device=dev),
                    pos_out=torch.full((U, B), -5, dtype=torch.int32, device=dev))
        plan = tri.PassPlan(c["K"], c["V"], c["pos"], c["row_off"], max_rows, c["t"], c["mu"], wl.theta, B,
                            ws=tri.make_workspace(U, max_rows, dev),
                            scores=torch.empty(int(P["row_off"][-1]), dtype=torch.float32, device=dev), **outs)
        return plan, outs, c

    ref_plan, ref, _ = copy_plan()
    ref_plan.run()
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(device=dev) for _ in range(2)]
    plans = []
    for i in range(4):
        with torch.cuda.stream(streams[i % 2]):
            plans.append(copy_plan())
    torch.cuda.synchronize()
    for it in range(40):
        plans[it % 4][0].run()
    torch.cuda.synchronize()
    for i, (_, outs, _) in enumerate(plans):
        for k in ref:
            assert torch.equal(outs[k], ref[k]), (i, k)


def test_c3_full_size_sampled():
    """All 288 units launched; the oracle checks a sample that includes near-zero-center units;
    select self-consistency and compaction are checked on every unit."""
    from synthgen.gen import flat_units

    wl = workload("c3")
    say("case c3: 288 x 32768 bf16 keys, B=2048 (generating)")
    P = pack_units(wl, workers=gen_workers())
    say("c3 generated; running")
    out = run_gpu(P, wl, wl.budget)
    flats = flat_units(wl)
    sample = sorted(set(flats[:3].tolist()) | {0, 143, 287})
    worst, total = 0.0, 0
    for i in range(wl.n_units):
        a, b = P["row_off"][i], P["row_off"][i + 1]
        if i in sample:
            err, mism = check_unit(P, i, wl, out, wl.budget, label="c3")
            worst, total = max(worst, err), total + mism
            say(f"c3 unit {i} flat={i in set(flats.tolist())}: err {err:.3g} mismatches {mism}")
        else:
            kept = out["kept_idx"][i, :wl.budget]
            assert out["kept_cnt"][i] == wl.budget
            assert np.array_equal(kept, O.select_topb(out["scores"][a:b], wl.budget)), i
            assert np.array_equal(out["K_out"][i], P["keys"][a:b][kept]), i
    say(f"c3 worst sampled score err {worst:.3g}")
    margin("C3 sample (288 x 32768 bf16, B=2048; 3 near-zero-center units among them)", worst, total, len(sample))


@pytest.mark.parametrize("max_rows", [None, SPLIT_ROWS])
def test_edge_cases_ragged_units(max_rows):
    """Empty, one-row, tail-sized and multi-chunk units in one launch; budgets 0, 1, between,
    equal to and above the unit sizes."""
    wl = workload("c2")
    lengths = [0, 1, 5, 511, 512, 513, 2049, 4100, 20000]
    units = list(range(len(lengths)))
    P = pack_units(dataclasses.replace(wl, heads=len(lengths)), units, lengths)
    for B in [0, 1, 300, 2048, 5000]:
        say(f"case edge ragged B={B} max_rows={max_rows}")
        out = run_gpu(P, wl, B, max_rows=max_rows)
        for i in range(len(lengths)):
            check_unit(P, i, wl, out, B, label=f"edge B={B}")
        assert out["ws_after"]


def test_granules_beyond_2_22_rows():
    """max_rows above 2^22 (an upper bound only; the units are short): granules of 2^11 rows and
    candidate chunks of two 1024-row tiles, through the pass and through the standalone select.
    Exact against the top-B of the GPU's own scores, bit for bit equal to the same pass at the
    natural max_rows, and the workspace back at rest."""
    wl = workload("c2")
    lengths = [0, 1, 5, 2049, 4100, 20000, 70000]
    units = list(range(len(lengths)))
    P = pack_units(dataclasses.replace(wl, heads=len(lengths)), units, lengths, workers=gen_workers())
    big = (1 << 22) + 1
    for B in [1, 300, 2048, 5000]:
        say(f"case max_rows=2^22+1 B={B}")
        ref = run_gpu(P, wl, B)
        for path in ["fused", "standalone"]:
            out = run_gpu(P, wl, B, max_rows=big, path=path)
            for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
                assert np.array_equal(out[k], ref[k]), (B, path, k)
            assert out["ws_after"], (B, path)
        for i in range(len(lengths)):
            check_unit(P, i, wl, out, B, label=f"max_rows=2^22+1 B={B}")


def test_many_units_one_workgroup_select():
    """396 ragged units (empty, one row, tails, up to 20000 rows): from 48 units and 384 groups of
    64 output slots on (every budget here, B = 0 and 1 included), the select holds each unit's
    keys in one workgroup and the compaction runs as its own kernel. Its results equal those of
    the fused resolve-and-emit path (max_rows above 64Ki) bit for bit, and sampled units match
    the oracle."""
    wl = workload("c2")
    pattern = [0, 1, 5, 511, 512, 513, 2049, 4100, 20000, 300, 64]
    lengths = pattern * 36
    units = list(range(len(lengths)))
    P = pack_units(dataclasses.replace(wl, heads=len(lengths)), units, lengths, workers=gen_workers())
    for B in [0, 1, 300, 2048, 5000]:
        say(f"case many units B={B}")
        out = run_gpu(P, wl, B)
        ref = run_gpu(P, wl, B, max_rows=65537)
        for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
            assert np.array_equal(out[k], ref[k]), (B, k)
        assert out["ws_after"]
        if B in (1, 2048):  # the three calls, and the standalone select with its own histogram
            for path in ["calls", "standalone"]:
                o2 = run_gpu(P, wl, B, path=path)
                for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
                    assert np.array_equal(o2[k], out[k]), (B, path, k)
                assert o2["ws_after"], (B, path)
        for i in [0, 1, 3, 8, 19, 263, 395]:
            check_unit(P, i, wl, out, B, label=f"many units B={B}")


def test_six_layers_in_one_call():
    """Six layers of the one-layer shape in one call (48 units of 32768 keys), the smallest unit
    count at which the select may hold each unit's keys in one workgroup: with B = 2048 (1536
    groups of 64 output slots) it does, with B = 256 (192 groups) the candidate and finish kernels
    run. Both equal, bit for bit, the same pass taken through candidates and finish by a max_rows
    above 64Ki, and sampled units match the oracle."""
    wl = dataclasses.replace(workload("c2"), layers=6)
    P = pack_units(wl, workers=gen_workers())
    for B in [256, 2048]:
        say(f"case six layers in one call B={B}")
        out = run_gpu(P, wl, B)
        ref = run_gpu(P, wl, B, max_rows=65537)
        for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
            assert np.array_equal(out[k], ref[k]), (B, k)
        assert out["ws_after"] and ref["ws_after"]
        for i in [0, 9, 30, 47]:
            check_unit(P, i, wl, out, B, label=f"six layers B={B}")


@pytest.mark.parametrize("n_units", [130, 520])
def test_candidate_workgroups_with_several_chunks(n_units):
    """With max_rows above 2^18 a unit has 257 candidate chunks of 1024 rows; past 16384 chunks in
    all, one candidate workgroup takes several consecutive chunks of its unit (4 for 130 units,
    16 for 520). Ragged units end inside a chunk and inside a workgroup's run of chunks. The
    results equal the bits of the one-workgroup-per-unit select (both unit counts are 48 or
    more, with 384 output groups or more), and sampled units match the oracle."""
    wl = workload("c2")
    pattern = [0, 1, 1023, 1024, 1025, 2049, 3000, 4097, 5000, 700]
    lengths = (pattern * (n_units // len(pattern) + 1))[:n_units]
    P = pack_units(dataclasses.replace(wl, heads=n_units), list(range(n_units)), lengths, workers=gen_workers())
    for B in [300, 2048]:
        say(f"case several chunks per candidate workgroup, {n_units} units, B={B}")
        out = run_gpu(P, wl, B, max_rows=SPLIT_ROWS)
        ref = run_gpu(P, wl, B)
        for k in ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]:
            assert np.array_equal(out[k], ref[k]), (B, k)
        assert out["ws_after"]
        for i in [2, 7, 8, n_units - 2]:
            check_unit(P, i, wl, out, B, label=f"chunks {n_units} B={B}")


def test_all_units_empty():
    """No rows at all (zero-size inputs): every unit keeps nothing, outputs stay untouched."""
    wl = dataclasses.replace(workload("c2"), heads=3)
    P = pack_units(wl, [0, 1, 2], [0, 0, 0])
    say("case all units empty")
    for path in ["fused", "calls", "standalone"]:
        out = run_gpu(P, wl, 16, path=path)
        assert np.all(out["kept_cnt"] == 0) and np.all(out["kept_idx"] == -1), path
        assert np.all(out["pos_out"] == -5), path
        assert out["ws_after"], path


def test_zero_center_all_ties():
    """A zero center scores every key +-0: the kept rows are the first B (lower-index rule)."""
    wl = workload("c2")
    P = pack_units(wl, [0, 1], [3000, 70])
    centers = P["centers"].copy()
    centers[0] = 0.0
    say("case zero center")
    out = run_gpu(P, wl, 1000, centers=centers)
    assert np.all(out["scores"][:3000] == 0)
    assert np.array_equal(out["kept_idx"][0], np.arange(1000))
    s_ref, scale = oracle_unit(P, 1, wl, centers=centers)
    check_unit(P, 1, wl, out, 1000, s_ref=s_ref, scale=scale, label="zero-center")


@pytest.mark.parametrize("long_len,max_rows", [(65536, None), (70000, None), (70000, SPLIT_ROWS)])
def test_zero_center_large_tie_group(long_len, max_rows):
    """40000 tied keys: more candidates than the candidate buffer holds (the paths that read the
    scores again instead), in the fused resolve-and-emit kernel and in the resolve kernel."""
    wl = workload("c2")
    P = pack_units(wl, [0, 1, 2], [40000, 9000, long_len])
    centers = P["centers"].copy()
    centers[0] = 0.0
    centers[2] = 0.0
    say(f"case zero center, 40000 and {long_len} ties, max_rows={max_rows}")
    for path in ["fused", "calls"]:
        out = run_gpu(P, wl, 2048, centers=centers, path=path, max_rows=max_rows)
        assert np.array_equal(out["kept_idx"][0], np.arange(2048))
        assert np.array_equal(out["kept_idx"][2], np.arange(2048))
        s_ref, scale = oracle_unit(P, 1, wl, centers=centers)
        check_unit(P, 1, wl, out, 2048, s_ref=s_ref, scale=scale, label=f"zero-center-large {path}")
        assert out["ws_after"]


@pytest.mark.parametrize("max_rows", [None, SPLIT_ROWS])
def test_quantized_scores_heavy_ties(max_rows):
    """Keys drawn from few values so that many scores tie exactly; kept rows must follow the
    lower-index rule across chunk boundaries."""
    wl = dataclasses.replace(workload("c2"), heads=2)
    P = pack_units(wl, [0, 1], [50000, 7000])
    rng = np.random.default_rng(33)
    from synthgen import f32_to_bf16_bits
    P["keys"] = f32_to_bf16_bits(rng.choice([-1.0, 0.5, 2.0], size=P["keys"].shape).astype(np.float32))
    P["pos"] = np.zeros_like(P["pos"])  # one distance: scores depend on the key only
    say(f"case quantized keys max_rows={max_rows}")
    for path in ["fused", "calls"]:
        out = run_gpu(P, wl, 3000, path=path, max_rows=max_rows)
        for i in range(2):
            check_unit(P, i, wl, out, 3000, label=f"quantized {path}")


@pytest.mark.parametrize("max_rows", [None, SPLIT_ROWS])
def test_dense_candidate_workgroup(max_rows):
    """1100 rows of one unit share one key and one position, so their scores tie exactly, and the
    budget puts the threshold inside that group: one candidate workgroup holds many more
    candidates than the resolve kernel preloads per workgroup, and the tie group is longer than
    its tie list."""
    wl = dataclasses.replace(workload("c2"), heads=1)
    P = pack_units(wl, [0], [20000])
    P["keys"][5000:6100] = P["keys"][5000]
    P["pos"][5000:6100] = P["pos"][5000]
    s_ref, scale = oracle_unit(P, 0, wl)
    above = int(np.sum(s_ref > s_ref[5000]))
    say(f"case dense candidate workgroup ({above} rows above the tie group) max_rows={max_rows}")
    for extra in [1, 550, 1100]:
        B = above + extra
        out = run_gpu(P, wl, B, max_rows=max_rows)
        check_unit(P, 0, wl, out, B, s_ref=s_ref, scale=scale, label=f"dense-cand +{extra}")
        nc, per_group, tie22 = candidate_profile(out["scores"], B)
        if extra < 1100:  # the threshold is the tie group's score
            assert nc <= 4096 and per_group > 256 and tie22 > 1024, (nc, per_group, tie22)
        kept = set(out["kept_idx"][0, :B].tolist())
        tied = [r for r in range(5000, 6100) if r in kept]
        assert tied == list(range(5000, 5000 + len(tied))), "ties keep the lowest rows"


@pytest.mark.parametrize("max_rows", [None, SPLIT_ROWS])
def test_candidate_overflow_spread_digits(max_rows):
    """Keys near one common key and one position crowd 60000 scores into a few top-digit bins:
    up to 13571 candidates, more than LDS holds, with digits 2 and 3 spread (the passes over
    the stored candidate words), and up to 277 candidates in one candidate workgroup (past the
    preloaded share)."""
    from synthgen import f32_to_bf16_bits

    wl = dataclasses.replace(workload("c2"), heads=2)
    P = pack_units(wl, [0, 1], [60000, 5000])
    rng = np.random.default_rng(41)
    k0 = rng.standard_normal(wl.d)
    P["keys"] = f32_to_bf16_bits((k0[None, :] + 0.05 * rng.standard_normal(P["keys"].shape)).astype(np.float32))
    P["pos"] = np.zeros_like(P["pos"])  # one distance: scores depend on the key only
    refs = [oracle_unit(P, i, wl) for i in range(2)]
    for B in [3000, 12000, 20000]:
        for path in ["fused", "calls"]:
            say(f"case candidate overflow B={B} {path} max_rows={max_rows}")
            out = run_gpu(P, wl, B, path=path, max_rows=max_rows)
            for i in range(2):
                check_unit(P, i, wl, out, B, s_ref=refs[i][0], scale=refs[i][1], label=f"overflow {path}")
            assert out["ws_after"]
            nc, per_group, _ = candidate_profile(out["scores"][:60000], B)
            if B > 3000:
                assert nc > 4096 and per_group > 128, (nc, per_group)


def test_very_long_unit():
    """One unit of 1.1 M rows: more than 1024 candidate workgroups and 512-row granules (eight
    emit steps per wave), with small and large budgets."""
    wl = dataclasses.replace(workload("c2"), heads=1)
    n = 1_100_000
    say("case very long unit (generating)")
    P = pack_units(wl, [0], [n])
    s_ref, scale = oracle_unit(P, 0, wl)
    for B in [100, 5000, 200000]:
        say(f"case very long unit B={B}")
        out = run_gpu(P, wl, B)
        check_unit(P, 0, wl, out, B, s_ref=s_ref, scale=scale, label=f"long B={B}")
        assert out["ws_after"]
        nc, _, _ = candidate_profile(out["scores"], B)
        say(f"   candidates {nc}")
        if B == 100:  # staged in LDS, one thread per candidate workgroup
            assert nc <= 4096, nc


def _rotated_case(wl, units, lengths, layout):
    """Generated keys rotated at their positions in fp64 and stored (rounded) in wl.dtype, with
    the oracle's post-rotation scores of the stored keys."""
    from synthgen import f32_to_bf16_bits

    P = pack_units(wl, units, lengths)
    omega = O.rotary_frequencies(wl.d, wl.theta)
    D = O.power_of_two_offsets()
    F = wl.d // 2
    lay = "half_split" if layout & 1 else "interleaved"
    stored = np.empty_like(P["keys"])
    refs = []
    for i in range(len(units)):
        a, b = P["row_off"][i], P["row_off"][i + 1]
        kb = O.as_bands(widen(P["keys"][a:b], wl.dtype))  # generated keys, interleaved bands
        kr = O.rotate_keys(kb, P["pos"][a:b], omega)
        x = np.empty((b - a, wl.d), dtype=np.float64)
        if lay == "interleaved":
            x[:, 0::2], x[:, 1::2] = kr.real, kr.imag
        else:
            x[:, :F], x[:, F:] = kr.real, kr.imag
        x32 = x.astype(np.float32)
        stored[a:b] = f32_to_bf16_bits(x32) if wl.dtype == "bf16" else x32
        ks = O.as_bands(widen(stored[a:b], wl.dtype), lay)  # what the kernel reads
        mu = O.folded_center(O.as_bands(P["centers"][i].astype(np.float64)), O.fold_weights(omega, D))
        s_ref = O.score_post_rope(mu, ks, int(P["t"][i]), omega)
        scale = np.sum(np.abs(mu)[None, :] * np.abs(ks), axis=1) / F
        refs.append((s_ref, scale))
    P["keys"] = stored
    return P, refs


@pytest.mark.parametrize("dtype,layout", [("bf16", 0), ("bf16", 1), ("f32", 0)])
def test_rotated_keys(dtype, layout):
    """Keys stored after the rotary rotation: the score from one coefficient vector per unit
    (mu' e^{i omega t}) against the oracle's post-rotation form of the same stored keys; the
    score alone, called without positions, gives the same bits."""
    import rotary_frequency_key_amd as tri

    wl = dataclasses.replace(workload("c2"), dtype=dtype, heads=3)
    P, refs = _rotated_case(wl, [0, 1, 2], [5000, 1500, 33], layout)
    say(f"case rotated keys {dtype} layout {layout}")
    out = run_gpu(P, wl, 700, layout=layout | tri.TRI_KEYS_ROTATED)
    worst, total = 0.0, 0
    for i in range(3):
        s_ref, scale = refs[i]
        err, mism = check_unit(P, i, wl, out, 700, s_ref=s_ref, scale=scale, label=f"rotated {dtype} {layout}")
        worst, total = max(worst, err), total + mism
    margin(f"rotated keys ({dtype}, {'half-split' if layout else 'interleaved'}; 5000/1500/33 rows, B=700)",
           worst, total, 3)
    dev = torch.device("cuda:0")
    from tests._parity import keys_to_device
    alone = tri.tri_score(keys_to_device(P["keys"], dtype, dev), torch.from_numpy(P["row_off"]).to(dev),
                          int(np.diff(P["row_off"]).max()), None, torch.from_numpy(P["t"]).to(dev),
                          torch.from_numpy(out["mu"]).to(dev), wl.theta, layout=layout | tri.TRI_KEYS_ROTATED)
    torch.cuda.synchronize()
    assert np.array_equal(alone.cpu().numpy(), out["scores"])


@pytest.mark.parametrize("d,dtype,layout", [(128, "bf16", 0), (128, "bf16", 1), (128, "f32", 0), (64, "f32", 0),
                                             (256, "bf16", 0)])
def test_max_over_offsets(d, dtype, layout):
    """The maximum over the offsets of the unfolded score, against the oracle's literal loop; then
    the select and the compaction on its histogram (score_max -> select -> compact), and the fused
    pass (tri_prune_pass_max), which must give the same bits. d = 128 runs on the matrix cores:
    17 offsets (one full tile of 16 and one padded), 5 (one padded tile) and 32 (two full tiles)."""
    import rotary_frequency_key_amd as tri

    wl = dataclasses.replace(workload("c2"), d=d, dtype=dtype, heads=3, theta=5e5)
    P = pack_units(wl, [0, 1, 2], [4000, 1500, 33])
    keys = P["keys"]
    F = d // 2
    if layout == 1:  # the same bands stored half-split
        perm = np.empty(d, dtype=int)
        perm[0::2] = np.arange(F)
        perm[1::2] = np.arange(F) + F
        keys = np.empty_like(P["keys"])
        keys[:, perm] = P["keys"]
    dev = torch.device("cuda:0")
    from tests._parity import keys_to_device, keys_to_host
    U, B = 3, 500
    sets = [O.power_of_two_offsets(), np.array([0, 3, 17, 1000, 99991], dtype=np.int64)]
    if d == 128:
        sets.append(np.arange(32, dtype=np.int64) * 977 + 5)
    for offsets in sets:
        say(f"case max over offsets d={d} {dtype} layout={layout} |D|={offsets.size}")
        K = keys_to_device(keys, dtype, dev)
        V = keys_to_device(P["values"], dtype, dev)
        pos = torch.from_numpy(P["pos"]).to(dev)
        row_off = torch.from_numpy(P["row_off"]).to(dev)
        t = torch.from_numpy(P["t"]).to(dev)
        centers = torch.from_numpy(np.ascontiguousarray(P["centers"], dtype=np.float32)).to(dev)
        ws = tri.make_workspace(U, 4000, dev)
        scores = tri.tri_score_max(K, row_off, 4000, pos, t, centers, wl.theta, offsets, layout=layout, ws=ws)
        kept_idx, kept_cnt = tri.tri_select_topb(scores, row_off, 4000, B, ws=ws, hist_from_score=True)
        K_out, V_out, pos_out = tri.tri_compact_kv(K, V, pos, row_off, kept_idx, kept_cnt, B)
        wsf = tri.make_workspace(U, 4000, dev)
        fused = tri.prune_pass_max(K, V, pos, row_off, 4000, t, centers, wl.theta, offsets, B, ws=wsf,
                                   layout=layout)
        torch.cuda.synchronize()
        for x, y, name in zip(fused[:3], (scores, kept_idx, kept_cnt), ("scores", "kept_idx", "kept_cnt")):
            assert torch.equal(x, y), f"fused pass: {name}"
        cnt = kept_cnt.cpu().numpy()
        for x, y, name in zip(fused[3:], (K_out, V_out, pos_out), ("K_out", "V_out", "pos_out")):
            xb, yb = x.cpu(), y.cpu()
            if xb.dtype == torch.bfloat16:
                xb, yb = xb.view(torch.int16), yb.view(torch.int16)
            for i in range(U):  # the kept rows; the slots past kept_cnt are not written
                assert torch.equal(xb[i, :cnt[i]], yb[i, :cnt[i]]), f"fused pass: {name}, unit {i}"
        assert ws_rest(wsf)
        s_gpu = scores.cpu().numpy()
        kept_all, K_out = kept_idx.cpu().numpy(), keys_to_host(K_out, dtype)
        assert ws_rest(ws)
        omega = O.rotary_frequencies(d, wl.theta)
        worst, total = 0.0, 0
        for i in range(U):
            a, b = P["row_off"][i], P["row_off"][i + 1]
            kb = O.as_bands(widen(P["keys"][a:b], dtype))
            cb = O.as_bands(P["centers"][i].astype(np.float64))
            s_ref = O.score_unfolded_max(cb, kb, O.distances(int(P["t"][i]), P["pos"][a:b]), omega, offsets)
            scale = np.sum(np.abs(cb)[None, :] * np.abs(kb), axis=1) / F
            err = score_error(s_gpu[a:b], s_ref, scale)
            say(f"   unit {i}: max score error {err:.3g}")
            assert err <= TOL, err
            m = min(B, b - a)
            kept = kept_all[i, :m]
            assert np.array_equal(kept, O.select_topb(s_gpu[a:b], B))
            from tests._parity import kept_mismatch
            worst, total = max(worst, err), total + kept_mismatch(kept, s_ref, scale, B)
            assert np.array_equal(K_out[i, :m], keys[a:b][kept])
        margin(f"max over offsets (d={d}, {dtype}, {'half-split' if layout else 'interleaved'}, |D|={offsets.size})",
               worst, total, U)


@pytest.mark.parametrize("d,dtype,layout", [(128, "bf16", 0), (128, "bf16", 1), (128, "f32", 0), (64, "f32", 0),
                                             (256, "bf16", 0)])
def test_max_over_offsets_rotated(d, dtype, layout):
    """Keys stored after the rotary rotation, maximum over the offsets. conj(k) e^{i w (t - p + delta)}
    = conj(k_rot) e^{i w (t + delta)}, so the reference is the oracle's literal loop on the stored
    keys with every distance equal to t. d = 128 is a bf16 matrix product of the key rows
    themselves; the scores are computed without positions. Then the fused pass
    (tri_prune_pass_max) against the three calls, bit for bit."""
    import rotary_frequency_key_amd as tri
    from tests._parity import kept_mismatch, keys_to_device, keys_to_host

    wl = dataclasses.replace(workload("c2"), d=d, dtype=dtype, heads=3, theta=5e5)
    P, _ = _rotated_case(wl, [0, 1, 2], [4000, 1500, 33], layout)
    lay = "half_split" if layout & 1 else "interleaved"
    F = d // 2
    U, B = 3, 500
    dev = torch.device("cuda:0")
    K = keys_to_device(P["keys"], dtype, dev)
    V = keys_to_device(P["values"], dtype, dev)
    pos = torch.from_numpy(P["pos"]).to(dev)
    row_off = torch.from_numpy(P["row_off"]).to(dev)
    t = torch.from_numpy(P["t"]).to(dev)
    centers = torch.from_numpy(np.ascontiguousarray(P["centers"], dtype=np.float32)).to(dev)
    omega = O.rotary_frequencies(d, wl.theta)
    rot = layout | tri.TRI_KEYS_ROTATED
    sets = [O.power_of_two_offsets(), np.array([0, 3, 17, 1000, 99991], dtype=np.int64)]
    if d == 128:
        sets.append(np.arange(32, dtype=np.int64) * 977 + 5)
    for offsets in sets:
        say(f"case max over offsets, rotated keys, d={d} {dtype} layout={layout} |D|={offsets.size}")
        ws = tri.make_workspace(U, 4000, dev)
        scores = tri.tri_score_max(K, row_off, 4000, None, t, centers, wl.theta, offsets, layout=rot, ws=ws)
        kept_idx, kept_cnt = tri.tri_select_topb(scores, row_off, 4000, B, ws=ws, hist_from_score=True)
        K_out, V_out, pos_out = tri.tri_compact_kv(K, V, pos, row_off, kept_idx, kept_cnt, B)
        wsf = tri.make_workspace(U, 4000, dev)
        fused = tri.prune_pass_max(K, V, pos, row_off, 4000, t, centers, wl.theta, offsets, B, ws=wsf, layout=rot)
        torch.cuda.synchronize()
        for x, y, name in zip(fused[:3], (scores, kept_idx, kept_cnt), ("scores", "kept_idx", "kept_cnt")):
            assert torch.equal(x, y), f"fused pass: {name}"
        cnt = kept_cnt.cpu().numpy()
        for x, y, name in zip(fused[3:], (K_out, V_out, pos_out), ("K_out", "V_out", "pos_out")):
            xb, yb = x.cpu(), y.cpu()
            if xb.dtype == torch.bfloat16:
                xb, yb = xb.view(torch.int16), yb.view(torch.int16)
            for i in range(U):
                assert torch.equal(xb[i, :cnt[i]], yb[i, :cnt[i]]), f"fused pass: {name}, unit {i}"
        assert ws_rest(ws) and ws_rest(wsf)
        s_gpu = scores.cpu().numpy()
        kept_all, K_host = kept_idx.cpu().numpy(), keys_to_host(K_out, dtype)
        worst, total = 0.0, 0
        for i in range(U):
            a, b = P["row_off"][i], P["row_off"][i + 1]
            ks = O.as_bands(widen(P["keys"][a:b], dtype), lay)  # the stored keys, as the kernel reads them
            cb = O.as_bands(P["centers"][i].astype(np.float64))
            dist = O.distances(int(P["t"][i]), np.zeros(b - a, dtype=np.int32))
            s_ref = O.score_unfolded_max(cb, ks, dist, omega, offsets)
            scale = np.sum(np.abs(cb)[None, :] * np.abs(ks), axis=1) / F
            err = score_error(s_gpu[a:b], s_ref, scale)
            say(f"   unit {i}: max score error {err:.3g}")
            assert err <= TOL, err
            m = min(B, b - a)
            kept = kept_all[i, :m]
            assert np.array_equal(kept, O.select_topb(s_gpu[a:b], B))
            worst, total = max(worst, err), total + kept_mismatch(kept, s_ref, scale, B)
            assert np.array_equal(K_host[i, :m], P["keys"][a:b][kept])
        margin(f"max over offsets, rotated keys (d={d}, {dtype}, {'half-split' if layout else 'interleaved'}, "
               f"|D|={offsets.size})", worst, total, U)


def test_max_pass_edge_cases():
    """The max-over-offsets pass on empty, one-row, tail-sized and multi-chunk units (up to 70000
    rows, beyond 2^16) in one launch, budgets 0, 1, 600 and above every unit, plain and rotated
    keys: the fused pass bit for bit against the three calls, both workspaces back at rest, the
    scores against the oracle's literal loop and the kept set the top-B of the GPU's scores."""
    import rotary_frequency_key_amd as tri
    from tests._parity import keys_to_device

    wl = workload("c2")
    lengths = [0, 1, 5, 511, 513, 4100, 70000]
    U, max_rows = len(lengths), max(lengths)
    P = pack_units(dataclasses.replace(wl, heads=U), list(range(U)), lengths, workers=gen_workers())
    dev = torch.device("cuda:0")
    K, V = keys_to_device(P["keys"], "bf16", dev), keys_to_device(P["values"], "bf16", dev)
    pos = torch.from_numpy(P["pos"]).to(dev)
    row_off = torch.from_numpy(P["row_off"]).to(dev)
    t = torch.from_numpy(P["t"]).to(dev)
    centers = torch.from_numpy(np.ascontiguousarray(P["centers"], dtype=np.float32)).to(dev)
    offsets = O.power_of_two_offsets()
    omega = O.rotary_frequencies(wl.d, wl.theta)
    F = wl.d // 2
    hist_words = U * 4096
    for layout in [0, tri.TRI_KEYS_ROTATED]:
        checked = False
        for B in [0, 1, 600, 80000]:
            say(f"case max pass edge units layout={layout:#x} B={B}")
            ws = tri.make_workspace(U, max_rows, dev)
            scores = tri.tri_score_max(K, row_off, max_rows, pos, t, centers, wl.theta, offsets, layout=layout, ws=ws)
            kept_idx, kept_cnt = tri.tri_select_topb(scores, row_off, max_rows, B, ws=ws, hist_from_score=True)
            K_out, V_out, pos_out = tri.tri_compact_kv(K, V, pos, row_off, kept_idx, kept_cnt, B)
            wsf = tri.make_workspace(U, max_rows, dev)
            fused = tri.prune_pass_max(K, V, pos, row_off, max_rows, t, centers, wl.theta, offsets, B, ws=wsf,
                                       layout=layout)
            torch.cuda.synchronize()
            for x, y, name in zip(fused[:3], (scores, kept_idx, kept_cnt), ("scores", "kept_idx", "kept_cnt")):
                assert torch.equal(x, y), f"fused pass: {name}"
            cnt = kept_cnt.cpu().numpy()
            for x, y, name in zip(fused[3:], (K_out, V_out, pos_out), ("K_out", "V_out", "pos_out")):
                xb, yb = x.cpu(), y.cpu()
                if xb.dtype == torch.bfloat16:
                    xb, yb = xb.view(torch.int16), yb.view(torch.int16)
                for i in range(U):
                    assert torch.equal(xb[i, :cnt[i]], yb[i, :cnt[i]]), f"fused pass: {name}, unit {i}"
            for w in (ws, wsf):
                assert bool(np.all(w[:hist_words * 4].cpu().numpy() == 0))
            s_gpu = scores.cpu().numpy()
            kept_all = kept_idx.cpu().numpy()
            for i in range(U):
                a, b = P["row_off"][i], P["row_off"][i + 1]
                m = min(B, b - a)
                assert cnt[i] == m
                assert np.array_equal(kept_all[i, :m], O.select_topb(s_gpu[a:b], B))
                assert np.all(kept_all[i, m:] == -1)
                if not checked and b > a:  # the scores do not depend on B: against the oracle once
                    kb = O.as_bands(widen(P["keys"][a:b], "bf16"))
                    cb = O.as_bands(P["centers"][i].astype(np.float64))
                    p_eff = np.zeros(b - a, dtype=np.int32) if layout else P["pos"][a:b]
                    s_ref = O.score_unfolded_max(cb, kb, O.distances(int(P["t"][i]), p_eff), omega, offsets)
                    scale = np.sum(np.abs(cb)[None, :] * np.abs(kb), axis=1) / F
                    err = score_error(s_gpu[a:b], s_ref, scale)
                    assert err <= TOL, (layout, i, err)
            checked = True


def ws_rest(ws):
    return bool(np.all(ws[:3 * 4096 * 4].cpu().numpy() == 0))


def _top_digits(scores):
    """Bits 31..20 of the key that orders binary32 scores as the select ranks them (descending,
    -0 equal to +0, NaN below every number): NaN -> 0, +-0 -> 2^31, a positive score -> its bits
    with the sign bit set, a negative score -> its bits inverted."""
    b = scores.view(np.uint32).astype(np.uint64)
    mag = b & 0x7FFFFFFF
    key = np.where(b >> 31 == 1, (~b) & 0xFFFFFFFF, b | 0x80000000)
    key = np.where(mag == 0, 0x80000000, key)
    key = np.where(mag > 0x7F800000, 0, key)
    return (key >> 20).astype(np.int64)


@pytest.mark.parametrize("kind", ["folded", "rotated", "max"])
def test_score_histogram_counts(kind):
    """The top-digit histogram the score kernels add into the workspace (the select's first
    radix digit) equals, per unit and bin, a count over the scores they return; a second call
    adds the same counts again. Ragged units (0 to 20000 rows, tails inside a 1024-row chunk)
    and one zero-center unit, whose scores are all +-0 (one bin)."""
    import rotary_frequency_key_amd as tri
    from tests._parity import keys_to_device

    wl = workload("c2")
    lengths = [0, 1, 5, 1023, 1025, 4100, 20000, 3000]
    U = len(lengths)
    P = pack_units(dataclasses.replace(wl, heads=U), list(range(U)), lengths)
    P["centers"][7] = 0.0
    dev = torch.device("cuda:0")
    K = keys_to_device(P["keys"], wl.dtype, dev)
    pos = torch.from_numpy(P["pos"]).to(dev)
    row_off = torch.from_numpy(P["row_off"]).to(dev)
    t = torch.from_numpy(P["t"]).to(dev)
    max_rows = max(lengths)
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, O.power_of_two_offsets(), P["centers"])
    mu_d = torch.from_numpy(mu).to(dev)
    centers = torch.from_numpy(np.ascontiguousarray(P["centers"], dtype=np.float32)).to(dev)
    ws = torch.zeros(U * 4096 * 4, dtype=torch.uint8, device=dev)
    say(f"case score histogram counts, {kind}")

    def call():
        if kind == "folded":
            return tri.tri_score(K, row_off, max_rows, pos, t, mu_d, wl.theta, ws=ws)
        if kind == "rotated":  # the same stored rows read as rotated keys
            return tri.tri_score(K, row_off, max_rows, None, t, mu_d, wl.theta,
                                 layout=tri.TRI_KEYS_ROTATED, ws=ws)
        return tri.tri_score_max(K, row_off, max_rows, pos, t, centers, wl.theta, O.power_of_two_offsets(), ws=ws)

    scores = call().cpu().numpy()
    torch.cuda.synchronize()
    h1 = ws.view(torch.int32).cpu().numpy().reshape(U, 4096).astype(np.int64)
    expect = np.zeros((U, 4096), dtype=np.int64)
    for u in range(U):
        a, b = int(P["row_off"][u]), int(P["row_off"][u + 1])
        expect[u] = np.bincount(_top_digits(scores[a:b]), minlength=4096)
    assert np.array_equal(h1, expect)
    assert expect[7, 2048] == lengths[7]  # the zero-center unit: every score +-0
    again = call().cpu().numpy()
    torch.cuda.synchronize()
    assert np.array_equal(again.view(np.uint32), scores.view(np.uint32))
    h2 = ws.view(torch.int32).cpu().numpy().reshape(U, 4096).astype(np.int64)
    assert np.array_equal(h2, 2 * expect)


def test_half_split_layout_matches_interleaved():
    wl = workload("c2")
    P = pack_units(wl, [2, 6], [4000, 777])
    d = wl.d
    perm = np.empty(d, dtype=int)
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    keys_hs = np.empty_like(P["keys"])
    keys_hs[:, perm] = P["keys"]
    say("case half-split layout")
    a = run_gpu(P, wl, 500)
    b = run_gpu(P, wl, 500, keys=keys_hs, layout=1)
    assert np.array_equal(a["scores"], b["scores"])
    assert np.array_equal(a["kept_idx"], b["kept_idx"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_head_dims_and_dtypes(d, dtype):
    wl = dataclasses.replace(workload("c2"), d=d, dtype=dtype, heads=3, theta=5e5)
    P = pack_units(wl, [0, 1, 2], [1500, 3333, 64])
    say(f"case d={d} {dtype}")
    out = run_gpu(P, wl, 256)
    for i in range(3):
        check_unit(P, i, wl, out, 256, label=f"d={d} {dtype}")


def test_large_distances_and_offsets():
    """Positions far from t (distance up to 2^24 - 1) and an arbitrary offset schedule."""
    wl = dataclasses.replace(workload("c2"), heads=2)
    P = pack_units(wl, [0, 1], [2000, 2000])
    rng = np.random.default_rng(5)
    P["pos"] = rng.integers(0, 1 << 23, size=4000).astype(np.int32)
    P["t"] = np.array([(1 << 24) - 1 + 0, (1 << 23) + 5], dtype=np.int32)
    P["pos"][0] = 0  # distance 2^24 - 1
    offsets = np.array([0, 3, 17, 1000, 99991], dtype=np.int64)
    say("case large distances")
    out = run_gpu(P, wl, 100, offsets=offsets, theta=1e4)
    for i in range(2):
        s_ref, scale = oracle_unit(P, i, wl, theta=1e4, offsets=offsets)
        check_unit(P, i, wl, out, 100, s_ref=s_ref, scale=scale, label="large-delta")


def test_select_standalone_special_values():
    """tri_select_topb on hand-made scores: NaN, +-0, +-inf, heavy ties, sizes spanning many
    blocks; bit-exact against the oracle's select."""
    import rotary_frequency_key_amd as tri

    dev = torch.device("cuda:0")
    rng = np.random.default_rng(21)
    lens = [0, 1, 7, 1024, 1025, 40000, 100003]
    parts = []
    for n in lens:
        s = rng.standard_normal(n).astype(np.float32)
        s[rng.random(n) < 0.3] = np.float32(0.5)  # a big tie group
        pick = rng.random(n)
        s[pick < 0.02] = np.nan
        s[(pick >= 0.02) & (pick < 0.04)] = -0.0
        s[(pick >= 0.04) & (pick < 0.06)] = 0.0
        s[(pick >= 0.06) & (pick < 0.07)] = np.inf
        s[(pick >= 0.07) & (pick < 0.08)] = -np.inf
        s[(pick >= 0.08) & (pick < 0.09)] = np.float32(1e-42)  # denormals
        parts.append(s)
    scores = np.concatenate(parts)
    row_off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    s_d = torch.from_numpy(scores).to(dev)
    r_d = torch.from_numpy(row_off).to(dev)
    for B in [0, 1, 3, 500, 1024, 30000, 200000]:
        say(f"case select special values B={B}")
        kept_idx, kept_cnt = tri.tri_select_topb(s_d, r_d, max(lens), B)
        torch.cuda.synchronize()
        kept_idx, kept_cnt = kept_idx.cpu().numpy(), kept_cnt.cpu().numpy()
        for i, n in enumerate(lens):
            ref = O.select_topb(scores[row_off[i]:row_off[i + 1]], B)
            assert kept_cnt[i] == ref.size
            assert np.array_equal(kept_idx[i, :ref.size], ref), (B, n)
            assert np.all(kept_idx[i, ref.size:] == -1)


def test_compact_skips_invalid_indices():
    import rotary_frequency_key_amd as tri

    dev = torch.device("cuda:0")
    wl = workload("c2")
    P = pack_units(wl, [0, 1], [100, 50])
    K = torch.from_numpy(P["keys"].view(np.int16)).to(dev).view(torch.bfloat16)
    V = torch.from_numpy(P["values"].view(np.int16)).to(dev).view(torch.bfloat16)
    pos = torch.from_numpy(P["pos"]).to(dev)
    row_off = torch.from_numpy(P["row_off"]).to(dev)
    kept = np.array([[3, -1, 99, 100, 7], [0, 49, 50, 2, 1]], dtype=np.int32)
    cnt = np.array([5, 3], dtype=np.int32)
    K_out = torch.full((2, 5, wl.d), 9.0, dtype=torch.bfloat16, device=dev)
    V_out = torch.full_like(K_out, 9.0)
    pos_out = torch.full((2, 5), -9, dtype=torch.int32, device=dev)
    say("case compact invalid indices")
    tri.tri_compact_kv(K, V, pos, row_off, torch.from_numpy(kept).to(dev), torch.from_numpy(cnt).to(dev), 5,
                       K_out=K_out, V_out=V_out, pos_out=pos_out)
    torch.cuda.synchronize()
    po = pos_out.cpu().numpy()
    assert po[0].tolist() == [3, -9, 99, -9, 7]
    assert po[1].tolist() == [0, 49, -9, -9, -9]
    ko = K_out.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ko[0, 2], P["keys"][99]) and np.array_equal(ko[1, 1], P["keys"][100 + 49])
