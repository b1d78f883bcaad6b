"""Workload recipes and the per-unit seeded generator.

A *unit* is one KV head of one layer of one sequence. Units are numbered
u = (seq * layers + layer) * heads + head and their rows are packed back to back in that order.

Recipe for unit (seq, layer, head) of a workload with seed s (one independent stream per unit,
so any unit can be regenerated alone):
  rng = numpy.random.default_rng([s, seq, layer, head])
  key center   mu_k  = rng.standard_normal(d) * 2
  query center q_c   = rng.standard_normal(d) * center_scale    (2, or 0.05 for a flat unit)
  keys         K     = mu_k + rng.standard_normal((N, d)) * key_sigma   (0.5, or 2.0 flat)
  values       V     = rng.standard_normal((N, d))
  everything drawn in float64, rounded to float32 (round-to-nearest-even), and K, V rounded
  again to bfloat16 (round-to-nearest-even) for bf16 workloads. Positions are 0..N-1 and the
  current position is t = N.

The workloads stand in for the long-reasoning and chat settings of the TriAttention README
(Qwen3-8B / Llama-3-8B / Qwen3-32B shapes, 32k context, budgets 2048 and 12000, 1024-token
prefill chunks); the public benchmark sets named there are not used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "workload",
    "f32_to_bf16_bits",
    "unit_lengths",
    "unit_inputs",
    "pack_units",
]


@dataclass(frozen=True)
class Workload:
    name: str
    seqs: int
    layers: int
    heads: int
    d: int
    dtype: str  # "f32" or "bf16"
    theta: float
    budget: int
    seed: int
    n_keys: int = 0  # keys per unit when every unit has the same length
    ragged: tuple = ()  # (lo, hi) inclusive: per-sequence lengths drawn uniformly
    flat_fraction: float = 0.0  # share of units with the near-zero center / wide-noise recipe
    key_sigma: float = 0.5
    center_scale: float = 2.0
    flat_key_sigma: float = 2.0
    flat_center_scale: float = 0.05
    description: str = ""

    @property
    def n_units(self) -> int:
        return self.seqs * self.layers * self.heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


WORKLOADS: Dict[str, Workload] = {
    "c1": Workload("c1", 1, 1, 1, 128, "f32", 1.0e4, 256, 1, n_keys=4096,
                   description="1 KV head, d=128, 4096 fp32 keys, theta=1e4, B=256"),
    "c2": Workload("c2", 1, 1, 8, 128, "bf16", 1.0e6, 2048, 2, n_keys=32768,
                   description="Qwen3-8B-shaped layer: 8 KV heads x 32768 bf16 keys, d=128, "
                               "theta=1e6, B=2048"),
    "c3": Workload("c3", 1, 36, 8, 128, "bf16", 1.0e6, 2048, 3, n_keys=32768, flat_fraction=0.1,
                   description="36 Qwen3-8B layers (288 units x 32768 keys), 10% of units with "
                               "a near-zero query center and sigma=2 key noise, B=2048"),
    "c4": Workload("c4", 16, 32, 8, 128, "bf16", 5.0e5, 2048, 4, ragged=(8192, 65536),
                   description="Llama-3-8B-shaped batch: 16 sequences x 32 layers x 8 KV heads, "
                               "lengths uniform in 8192..65536 per sequence, B=2048"),
    "c5": Workload("c5", 4, 64, 8, 128, "bf16", 1.0e6, 12000, 5, n_keys=131072 + 1024,
                   description="Qwen3-32B-shaped long context: 4 sequences x 64 layers x 8 KV "
                               "heads, 131072 keys + a 1024-key chunk, B=12000"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest, ties to even.

    Inputs are finite. The rounding adds 0x7FFF plus the lowest kept bit, then truncates.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((b >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((b + bias) >> np.uint32(16)).astype(np.uint16)


def unit_lengths(wl: Workload) -> np.ndarray:
    """Keys per unit, int64 [n_units]. Ragged workloads draw one length per sequence from the
    stream default_rng([seed, 0xFFFF]); all layers and heads of a sequence share it."""
    if wl.ragged:
        lo, hi = wl.ragged
        per_seq = np.random.default_rng([wl.seed, 0xFFFF]).integers(lo, hi, size=wl.seqs,
                                                                      endpoint=True)
        return np.repeat(per_seq.astype(np.int64), wl.layers * wl.heads)
    return np.full(wl.n_units, wl.n_keys, dtype=np.int64)


def flat_units(wl: Workload) -> np.ndarray:
    """Sorted ids of the units that use the near-zero-center recipe: the first
    round(flat_fraction * n_units) entries of a permutation drawn from default_rng([seed, 0xFFFE])."""
    n = int(round(wl.flat_fraction * wl.n_units))
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    perm = np.random.default_rng([wl.seed, 0xFFFE]).permutation(wl.n_units)
    return np.sort(perm[:n]).astype(np.int64)


def _unit_coords(wl: Workload, u: int):
    head = u % wl.heads
    layer = (u // wl.heads) % wl.layers
    seq = u // (wl.heads * wl.layers)
    return seq, layer, head


def unit_inputs(wl: Workload, u: int, n_keys: int | None = None, with_values: bool = True):
    """Inputs of unit u, as the device receives them.

    Returns dict(keys, values, center, pos, t): keys/values are uint16 bf16 bits or float32,
    shape [N, d]; center is float32 [d] (interleaved band pairs); pos int32 [N]; t int.
    """
    if n_keys is None:
        n_keys = int(unit_lengths(wl)[u])
    seq, layer, head = _unit_coords(wl, u)
    flat = u in set(flat_units(wl).tolist())
    rng = np.random.default_rng([wl.seed, seq, layer, head])
    d = wl.d
    key_center = rng.standard_normal(d) * 2.0
    center = rng.standard_normal(d) * (wl.flat_center_scale if flat else wl.center_scale)
    sigma = wl.flat_key_sigma if flat else wl.key_sigma
    keys64 = key_center[None, :] + rng.standard_normal((n_keys, d)) * sigma
    keys32 = keys64.astype(np.float32)
    del keys64
    if with_values:
        vals32 = rng.standard_normal((n_keys, d)).astype(np.float32)
    else:
        vals32 = None
    if wl.dtype == "bf16":
        keys = f32_to_bf16_bits(keys32)
        values = f32_to_bf16_bits(vals32) if vals32 is not None else None
    else:
        keys, values = keys32, vals32
    return {
        "keys": keys,
        "values": values,
        "center": center.astype(np.float32),
        "pos": np.arange(n_keys, dtype=np.int32),
        "t": int(n_keys),
    }


def _unit_job(args):
    wl, u, n = args
    return unit_inputs(wl, u, n)


def pack_units(wl: Workload, units: Sequence[int] | None = None, lengths: Sequence[int] | None = None,
               workers: int = 1):
    """Pack several units back to back; ``workers`` > 1 generates units in a process pool
    (spawned processes that only run this generator).

    Returns dict(keys [R, d], values [R, d], centers [U, d] float32, pos int32 [R],
    t int32 [U], row_off int64 [U+1], units list).
    """
    if units is None:
        units = list(range(wl.n_units))
    units = list(units)
    if lengths is None:
        all_len = unit_lengths(wl)
        lengths = [int(all_len[u]) for u in units]
    jobs = [(wl, u, int(n)) for u, n in zip(units, lengths)]
    if workers > 1 and len(jobs) > 1:
        import multiprocessing as mp
        from concurrent.futures import ProcessPoolExecutor

        with ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn")) as ex:
            parts: List[dict] = list(ex.map(_unit_job, jobs, chunksize=1))
    else:
        parts = [_unit_job(j) for j in jobs]
    row_off = np.zeros(len(units) + 1, dtype=np.int64)
    row_off[1:] = np.cumsum([p["keys"].shape[0] for p in parts])
    return {
        "keys": np.concatenate([p["keys"] for p in parts], axis=0),
        "values": np.concatenate([p["values"] for p in parts], axis=0),
        "centers": np.stack([p["center"] for p in parts], axis=0),
        "pos": np.concatenate([p["pos"] for p in parts]),
        "t": np.array([p["t"] for p in parts], dtype=np.int32),
        "row_off": row_off,
        "units": units,
    }
