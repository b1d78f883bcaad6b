"""tri_prune_pass_noalloc (the pass with the library's static workspace, for callers that cannot
allocate) against tri_prune_pass with a workspace of its own: every output bit for bit, over
consecutive calls that share the static array - the bench shape, then a smaller ragged batch,
then the bench shape again - through every select arrangement, captured in a HIP graph, and its
size limit and argument checks on the host."""
import ctypes
import os
import re

import numpy as np
import pytest

from synthgen import pack_units, workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = ["scores", "kept_idx", "kept_cnt", "K_out", "V_out", "pos_out"]


def say(*a):
    print("[no-alloc]", *a, flush=True)


def test_scratch_size_matches_header():
    import rotary_frequency_key_amd as tri

    hdr = open(os.path.join(ROOT, "include", "tri.h")).read()
    m = re.search(r"#define TRI_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == tri.NOALLOC_SCRATCH_BYTES


def test_rejects_passes_beyond_the_scratch_size():
    """Host only: a shape whose workspace exceeds the static array returns TRI_ERR_WORKSPACE
    before any HIP call (the fake device addresses are never used), and the limit sits where
    tri_prune_pass's size query puts it."""
    from rotary_frequency_key_amd import _abi

    lib = _abi._lib
    cap = _abi.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 40)

    def need(U, rows):
        n = ctypes.c_size_t(0)
        assert lib.tri_prune_pass(None, None, 1, 0, 128, 1e6, None, U, 0, rows, None, None, None, 2048, None,
                                  None, None, None, None, None, None, ctypes.byref(n), None) == 0
        return n.value

    def call(U, rows):
        return lib.tri_prune_pass_noalloc(fake, fake, 1, 0, 128, 1e6, fake, U, U * rows, rows, fake, fake, fake,
                                          2048, fake, fake, fake, fake, fake, fake, None)

    assert need(288, 32768) <= cap  # every layer of one sequence fits
    U = 1
    while need(U, 65536) <= cap:
        U *= 2
    assert call(U, 65536) == -4
    assert call(1, 1 << 30) == -4
    assert call(0, 1024) == -1 and call(1, -1) == -1 and call(1, 1 << 31) == -1


@pytest.mark.gpu
def test_noalloc_matches_prune_pass_on_consecutive_calls():
    import torch

    from tests._parity import check_unit, gen_workers, run_gpu

    wl = workload("c2")
    P_big = pack_units(wl, workers=gen_workers())
    P_small = pack_units(wl, [0, 1, 2, 3, 4], [0, 1, 3000, 9000, 20000])
    cases = [("8 x 32768, B=2048", P_big, wl.budget), ("5 ragged units (0..20000 rows), B=1000", P_small, 1000),
             ("8 x 32768, B=2048 again", P_big, wl.budget)]
    for name, P, B in cases:
        say(name)
        ref = run_gpu(P, wl, B)
        got = run_gpu(P, wl, B, path="noalloc")
        for k in KEYS:
            assert np.array_equal(got[k], ref[k]), (name, k)
        assert ref["ws_after"], name
    # the smaller call against the oracle as well
    out = run_gpu(P_small, wl, 1000, path="noalloc")
    for i in range(5):
        check_unit(P_small, i, wl, out, 1000, label="no-alloc ragged")
    torch.cuda.synchronize()


@pytest.mark.gpu
def test_noalloc_every_select_arrangement():
    """The static workspace through the other select arrangements, each against tri_prune_pass:
    264 ragged units (one workgroup per unit, then the compaction kernel), and ragged units and the
    8 x 32768 layer with max_rows above 2^18 (candidates, resolve, emit); the arrangements
    alternate, so each call starts from what a different one left in the array."""
    import dataclasses

    from tests._parity import SPLIT_ROWS, gen_workers, run_gpu

    wl = workload("c2")
    pattern = [0, 1, 5, 511, 512, 513, 2049, 4100, 20000, 300, 64]
    lengths = pattern * 24
    P = pack_units(dataclasses.replace(wl, heads=len(lengths)), list(range(len(lengths))), lengths,
                   workers=gen_workers())
    P8 = pack_units(wl, workers=gen_workers())
    P9 = pack_units(dataclasses.replace(wl, heads=9), list(range(9)), pattern[:9])
    # (264 units with max_rows above 2^18 would need more workspace than the static array holds)
    for name, PP, B, mr in [("264 ragged units, B=300", P, 300, None), ("8 x 32768", P8, wl.budget, None),
                            ("9 ragged units, max_rows 2^18+1, B=2048", P9, 2048, SPLIT_ROWS),
                            ("8 x 32768, max_rows 2^18+1", P8, wl.budget, SPLIT_ROWS),
                            ("264 ragged units, B=5000", P, 5000, None)]:
        say(name)
        ref = run_gpu(PP, wl, B, max_rows=mr)
        got = run_gpu(PP, wl, B, max_rows=mr, path="noalloc")
        for k in KEYS:
            assert np.array_equal(got[k], ref[k]), (name, k)


@pytest.mark.gpu
def test_noalloc_pass_in_a_graph():
    """The pass without a workspace captured in a HIP graph (torch.cuda.graph) and replayed four
    times, with eager work and synchronisations between replays: every replay equals the eager
    call bit for bit (the static array's address is taken by an eager call before the capture)."""
    import torch

    import rotary_frequency_key_amd as tri
    from tests._parity import gen_workers, keys_to_device

    dev = torch.device("cuda:0")
    wl = workload("c2")
    P = pack_units(wl, workers=gen_workers())
    U, B = wl.n_units, wl.budget
    max_rows = int(np.diff(P["row_off"]).max())
    _, mu = tri.tri_fold_weights(wl.d, wl.theta, np.array([1 << j for j in range(17)]), P["centers"])
    K, V = keys_to_device(P["keys"], "bf16", dev), keys_to_device(P["values"], "bf16", dev)
    pos = torch.from_numpy(P["pos"]).to(dev)
    row_off = torch.from_numpy(P["row_off"]).to(dev)
    t_now = torch.from_numpy(P["t"]).to(dev)
    mu_d = torch.from_numpy(mu).to(dev)
    R = K.shape[0]
    outs = dict(scores=torch.empty(R, dtype=torch.float32, device=dev),
                kept_idx=torch.empty((U, B), dtype=torch.int32, device=dev),
                kept_cnt=torch.empty(U, dtype=torch.int32, device=dev),
                K_out=torch.empty((U, B, wl.d), dtype=torch.bfloat16, device=dev),
                V_out=torch.empty((U, B, wl.d), dtype=torch.bfloat16, device=dev),
                pos_out=torch.empty((U, B), dtype=torch.int32, device=dev))

    def call():
        tri.prune_pass_noalloc(K, V, pos, row_off, max_rows, t_now, mu_d, wl.theta, B, **outs)

    s = torch.cuda.Stream(device=dev)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # eager, on the capture stream: the array's address is taken here, not under capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in outs.items()}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        for v in outs.values():
            v.zero_()
        scratch = torch.randn(1 << 20, device=dev)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in KEYS:
            a, b = outs[k], ref[k]
            if a.dtype == torch.bfloat16:
                a, b = a.view(torch.int16), b.view(torch.int16)
            assert torch.equal(a, b), (rep, k)
        del scratch
