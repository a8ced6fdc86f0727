"""Seeded synthetic inputs for the KV residency engine.

This package produces the inputs that both the CPU oracle and the HIP engine
consume: workload presets, decode-step selection traces, append schedules and
the contents of KV rows. It holds none of the replacement method's arithmetic
(no lookup, no bucket logic, no eviction): it only draws positions and bytes.

The workloads stand in for the long-document summarisation traces that the
UlaCache summary (paper-daily.com, "UlaCache: Unified Logical Addressing for
Sparse LLM Serving", section 4) measures on: contexts of 64K-128K tokens,
sparse top-k selection with heavy step-to-step overlap (section 2), and
656-byte MLA rows stored in FP8 (sections 1 and 4). No dataset item is used.
"""

from .configs import Workload, PRESETS, preset, scaled
from .traces import Trace
from .rows import splitmix64, rows_for, row

__all__ = ["Workload", "PRESETS", "preset", "scaled", "Trace", "splitmix64", "rows_for", "row"]
