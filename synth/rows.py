"""Contents of synthetic KV rows.

A row is ``row_bytes`` opaque bytes (the pages' FP8 MLA latent, bf16 rope and
scales; nothing in the engine interprets them). Row ``(g, la, l)`` is the
little-endian byte string of the words ``splitmix64(x_q)`` for
``q = 0 .. row_bytes/8 - 1`` with

    x_q = (seed << 56) ^ (g << 47) ^ (l << 39) ^ (la << 7) ^ q

which is injective for seed, g, l < 256, la < 2^31 and q < 128.

splitmix64 is the public-domain output function of Steele, Lea and Flood
("Fast splittable pseudorandom number generators", OOPSLA 2014) in the form
Sebastiano Vigna publishes with xoshiro: add the golden-ratio increment, then
two xor-shift-multiply rounds and a final xor-shift, all modulo 2^64.

A HIP implementation of the same definition lives in ``synth/csrc`` and fills
device buffers for the GPU side; the two are compared on sampled rows.
"""

from __future__ import annotations

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
MIX1 = np.uint64(0xBF58476D1CE4E5B9)
MIX2 = np.uint64(0x94D049BB133111EB)


def splitmix64(x: np.ndarray) -> np.ndarray:
    """splitmix64 output for state ``x`` (uint64 array, wraps mod 2^64)."""
    z = np.array(x, dtype=np.uint64, copy=True)
    return _splitmix64_inplace(z, np.empty_like(z))


def _splitmix64_inplace(z: np.ndarray, t: np.ndarray) -> np.ndarray:
    z += GOLDEN
    np.right_shift(z, np.uint64(30), out=t)
    z ^= t
    z *= MIX1
    np.right_shift(z, np.uint64(27), out=t)
    z ^= t
    z *= MIX2
    np.right_shift(z, np.uint64(31), out=t)
    z ^= t
    return z


def _check(seed: int, g: int, layers: int, row_bytes: int) -> None:
    if not (0 <= seed < 256 and 0 <= g < 256 and 0 < layers <= 256):
        raise ValueError("seed, group and layer must be below 256")
    if row_bytes % 8 or not (0 < row_bytes <= 1024):
        raise ValueError("row_bytes must be a multiple of 8 and at most 1024")


def rows_for(seed: int, g: int, las: np.ndarray, layers: int, row_bytes: int,
             chunk: int = 256) -> np.ndarray:
    """uint8 [n][layers][row_bytes]: the rows of every layer for each address."""
    _check(seed, g, layers, row_bytes)
    las = np.asarray(las, dtype=np.int64).reshape(-1)
    n, words = las.size, row_bytes // 8
    out = np.empty((n, layers, words), dtype=np.uint64)
    # low bits of x that do not depend on the address: layer and word index
    lw = ((np.arange(layers, dtype=np.uint64)[:, None] << np.uint64(39))
          ^ np.arange(words, dtype=np.uint64)[None, :])
    lw ^= (np.uint64(seed) << np.uint64(56)) ^ (np.uint64(g) << np.uint64(47))
    tmp = np.empty((chunk, layers, words), dtype=np.uint64)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        z = out[s:e]
        np.bitwise_xor(lw[None, :, :], (las[s:e].astype(np.uint64) << np.uint64(7))[:, None, None], out=z)
        _splitmix64_inplace(z, tmp[: e - s])
    return out.astype("<u8", copy=False).view(np.uint8).reshape(n, layers, row_bytes)


def row(seed: int, g: int, la: int, layer: int, row_bytes: int) -> np.ndarray:
    """uint8 [row_bytes] for one (group, address, layer)."""
    _check(seed, g, layer + 1, row_bytes)
    q = np.arange(row_bytes // 8, dtype=np.uint64)
    x = ((np.uint64(seed) << np.uint64(56)) ^ (np.uint64(g) << np.uint64(47))
         ^ (np.uint64(layer) << np.uint64(39)) ^ (np.uint64(la) << np.uint64(7)) ^ q)
    return splitmix64(x).astype("<u8").view(np.uint8)
