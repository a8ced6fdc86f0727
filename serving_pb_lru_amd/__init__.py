"""PB-LRU KV residency engine for MI355X (gfx950).

A per-decode-step residency layer for index-based sparse attention, in its
single-GPU (DP) form, after "UlaCache: Unified Logical Addressing for Sparse
LLM Serving" (paper-daily.com summary, sections 2 and 3): every logical KV
entry lives in exactly one of a GPU pool and a pinned host pool, a mapping
table tracks which, and PB-LRU (ring of per-round buckets plus a cold bucket,
bitmaps with summaries) picks what leaves the GPU. All of the per-step work
runs in hand-written HIP kernels behind the C ABI of include/ula.h; the
Python module `ula` only marshals arguments.
"""

from .ula import Engine, UlaError, lib, ERROR_NAMES

__all__ = ["Engine", "UlaError", "lib", "ERROR_NAMES"]
