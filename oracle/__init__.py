"""fp64 CPU oracle for the TriAttention key-eviction pass (score, top-B select, compaction).

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path (the HIP
library and its Python binding) never imports, links or calls anything here,
and this package imports nothing from the product path.

Sources, cited by page title and section:
  [N] "The future-offset average in TriAttention can be precomputed"
      (A. Mukherjee, July 2026), sections "The score TriAttention computes",
      "The same score, read as arrows in the plane", "The averaging step",
      "What it saves, and what it does not".
  [R] The TriAttention project README, sections on chat-mode settings
      (KV budget) and the headline claims.

Readings of points the pages leave open are listed in ``tri_oracle``'s
docstrings, marked "Reading".
"""
from .tri_oracle import *  # noqa: F401,F403
