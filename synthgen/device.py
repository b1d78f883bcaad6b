"""Full-size workloads generated on the device.

The largest workloads (4096 ragged units of 8192..65536 keys; 2048 units of 132096 keys) hold
77 GB and 138 GB of K and V: too much to draw on the host. This generator follows the same
recipe as gen.py (key center * 2, keys = center + noise * sigma, query center * scale, V
standard normal, positions 0..N-1, t = N) with the centers drawn on the host per unit
(default_rng([seed, seq, layer, head]), so they are the host recipe's) and the noise drawn on the
device with torch's generator seeded by (seed, block). The per-key values therefore differ from
gen.py's streams; the distribution, shapes and ragged lengths are the same. Nothing here
computes any part of the method.
"""
from __future__ import annotations

import numpy as np

from .gen import Workload, flat_units, unit_lengths

__all__ = ["device_workload"]


def _centers(wl: Workload):
    """Host per-unit key and query centers (the first two draws of gen.py's per-unit stream)."""
    flats = set(flat_units(wl).tolist())
    kc = np.empty((wl.n_units, wl.d), dtype=np.float32)
    qc = np.empty((wl.n_units, wl.d), dtype=np.float32)
    sig = np.empty(wl.n_units, dtype=np.float32)
    for u in range(wl.n_units):
        head = u % wl.heads
        layer = (u // wl.heads) % wl.layers
        seq = u // (wl.heads * wl.layers)
        rng = np.random.default_rng([wl.seed, seq, layer, head])
        kc[u] = rng.standard_normal(wl.d) * 2.0
        flat = u in flats
        qc[u] = rng.standard_normal(wl.d) * (wl.flat_center_scale if flat else wl.center_scale)
        sig[u] = wl.flat_key_sigma if flat else wl.key_sigma
    return kc, qc, sig


def device_workload(wl: Workload, device, block_rows: int = 1 << 22):
    """Return dict(K, V [R, d] device, pos int32 [R] device, row_off int64 [U+1] host and device,
    t int32 [U] host and device, centers float32 [U, d] host)."""
    import torch

    lengths = unit_lengths(wl)
    U = wl.n_units
    row_off = np.zeros(U + 1, dtype=np.int64)
    row_off[1:] = np.cumsum(lengths)
    R = int(row_off[-1])
    kc, qc, sig = _centers(wl)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    K = torch.empty((R, wl.d), dtype=dt, device=device)
    V = torch.empty((R, wl.d), dtype=dt, device=device)
    unit_of_row = torch.repeat_interleave(torch.arange(U, device=device), torch.from_numpy(lengths).to(device))
    kc_d = torch.from_numpy(kc).to(device)
    sig_d = torch.from_numpy(sig).to(device)
    g = torch.Generator(device=device)
    for b, r0 in enumerate(range(0, R, block_rows)):
        r1 = min(R, r0 + block_rows)
        g.manual_seed(int(wl.seed) * 1_000_003 + b)
        u = unit_of_row[r0:r1]
        noise = torch.randn((r1 - r0, wl.d), generator=g, device=device, dtype=torch.float32)
        K[r0:r1] = (kc_d[u] + noise * sig_d[u][:, None]).to(dt)
        V[r0:r1] = torch.randn((r1 - r0, wl.d), generator=g, device=device, dtype=torch.float32).to(dt)
        del noise, u
    starts = torch.from_numpy(row_off[:-1]).to(device)
    pos = (torch.arange(R, device=device, dtype=torch.int64) - starts[unit_of_row]).to(torch.int32)
    del unit_of_row
    t = lengths.astype(np.int32)
    return {"K": K, "V": V, "pos": pos, "row_off": row_off, "row_off_d": torch.from_numpy(row_off).to(device),
            "t": t, "t_d": torch.from_numpy(t).to(device), "centers": qc, "lengths": lengths}
