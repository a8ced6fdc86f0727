"""Digests of exported residency states (test infrastructure).

The same function digests the oracle's state (when the golden files are
written) and the engine's state (when the GPU tests compare against them).
"""

import numpy as np
import xxhash

FIELDS = ("map", "gown", "hown", "bitsets")
DTYPES = {"map": "<u4", "gown": "<i4", "hown": "<i4", "bitsets": "<u4"}


def digest(st: dict) -> dict:
    out = {}
    for k in FIELDS:
        a = np.ascontiguousarray(np.asarray(st[k]).astype(DTYPES[k], copy=False))
        out[k] = xxhash.xxh3_64_hexdigest(a.tobytes())
    out["cur"] = int(st["cur"])
    out["flag"] = int(st["flag"])
    out["stats"] = [int(x) for x in st["stats"]]
    if "stamps" in st:   # exact LRU's timestamps
        out["stamps"] = xxhash.xxh3_64_hexdigest(np.ascontiguousarray(
            np.asarray(st["stamps"]).astype("<i4", copy=False)).tobytes())
    return out
