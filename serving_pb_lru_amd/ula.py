"""Python binding of libula.so: argument marshalling only.

Every step of the residency path runs in the HIP kernels behind the C ABI in
include/ula.h; this module turns torch tensors and numpy arrays into pointers
and sizes, and error codes into exceptions. PyTorch supplies the device
workspace and the streams. There is no fallback: without the built library
every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libula.so")

ERROR_NAMES = {0: "OK", -1: "EINVAL", -2: "ERANGE", -3: "EDUP", -4: "EHOSTFULL",
               -5: "ECAPACITY", -6: "ENOTRESIDENT", -7: "ESTATE", -8: "EHIP", -9: "EBUSY",
               -10: "ETOOBIG"}


POLICY_PBLRU, POLICY_LRU = 0, 1
PLACE_LOWEST, PLACE_RING = 0, 1


class UlaConfig(ctypes.Structure):
    _fields_ = [("num_groups", ctypes.c_int32), ("layers_per_group", ctypes.c_int32),
                ("row_bytes", ctypes.c_int32), ("ring_buckets", ctypes.c_int32),
                ("logical_capacity", ctypes.c_int32), ("gpu_slots", ctypes.c_int32),
                ("host_slots", ctypes.c_int32), ("max_sets", ctypes.c_int32),
                ("max_k", ctypes.c_int32), ("max_append", ctypes.c_int32), ("policy", ctypes.c_int32),
                ("placement", ctypes.c_int32)]


class UlaStepStats(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in
                ("unique", "hits", "misses", "evictions", "from_free", "invalid")]

    def as_tuple(self):
        return (self.unique, self.hits, self.misses, self.evictions, self.from_free, self.invalid)


class UlaStateHost(ctypes.Structure):
    _fields_ = [("map", ctypes.c_void_p), ("gown", ctypes.c_void_p), ("hown", ctypes.c_void_p),
                ("bitsets", ctypes.c_void_p), ("cur", ctypes.c_int32), ("flag", ctypes.c_int64),
                ("last", UlaStepStats), ("stamps", ctypes.c_void_p)]


class UlaError(RuntimeError):
    def __init__(self, code: int, where: str, text: str):
        self.code = code
        self.name = ERROR_NAMES.get(code, str(code))
        super().__init__(f"{where}: {self.name} ({text})")


_lib = None

# (name, restype, argtypes) of every symbol include/ula.h declares
SIGNATURES = [
    ("ula_device_bytes", ctypes.c_size_t, [ctypes.POINTER(UlaConfig)]),
    ("ula_host_bytes", ctypes.c_size_t, [ctypes.POINTER(UlaConfig)]),
    ("ula_init", ctypes.c_int, [ctypes.POINTER(UlaConfig), ctypes.c_void_p, ctypes.c_void_p,
                                ctypes.c_uint64, ctypes.POINTER(ctypes.c_void_p)]),
    ("ula_init_static", ctypes.c_int, [ctypes.POINTER(UlaConfig), ctypes.c_void_p, ctypes.c_uint64,
                                       ctypes.POINTER(ctypes.c_void_p)]),
    ("ula_append", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64]),
    ("ula_release", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                   ctypes.c_uint64]),
    ("ula_step", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_void_p, ctypes.c_uint64]),
    ("ula_append_step", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_uint64]),
    ("ula_gather", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64]),
    ("ula_gather_layers", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_uint64]),
    ("ula_sync", ctypes.c_int, [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
    ("ula_export_state", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(UlaStateHost)]),
    ("ula_read_rows", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]),
    ("ula_flag_address", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_void_p)]),
    ("ula_set_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32]),
    ("ula_read_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]),
    ("ula_read_gather_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                              ctypes.POINTER(ctypes.c_int64)]),
    ("ula_read_link_timing", ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_double),
                                            ctypes.POINTER(ctypes.c_int64)]),
    ("ula_destroy", ctypes.c_int, [ctypes.c_void_p]),
    ("ula_strerror", ctypes.c_char_p, [ctypes.c_int]),
    ("ula_host_alloc", ctypes.c_void_p, [ctypes.c_size_t]),
    ("ula_host_free", ctypes.c_int, [ctypes.c_void_p]),
]


def lib() -> ctypes.CDLL:
    """Load libula.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with serving_pb_lru_amd.build.build()")
        # torch ships its own HIP runtime under the same soname as the one this
        # library links; importing torch first makes the library bind to that
        # runtime (loaded the other way round, the process ends up with two HIP
        # runtimes and device calls fail)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in SIGNATURES:
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise UlaError(rc, where, lib().ula_strerror(rc).decode())


def _dev(t, dtype: str, count: int, what: str) -> int:
    """Device pointer of a contiguous CUDA tensor of `dtype` holding at least
    `count` elements; raises ValueError otherwise (the library takes plain
    pointers and would read or write past a smaller buffer)."""
    if not (hasattr(t, "is_cuda") and t.is_cuda):
        raise ValueError(f"{what}: a CUDA tensor is required")
    if str(t.dtype) != f"torch.{dtype}":
        raise ValueError(f"{what}: dtype {t.dtype}, expected torch.{dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{what}: the tensor must be contiguous")
    if t.numel() < count:
        raise ValueError(f"{what}: {t.numel()} elements, at least {count} needed")
    return t.data_ptr()


def _sets(sel):
    """(n_sets, k) of a selection tensor [n_sets][k] or [k]."""
    return (1, sel.shape[0]) if sel.dim() == 1 else tuple(sel.shape)


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Engine:
    """One engine context: per group a GPU pool, a pinned host pool and PB-LRU state."""

    def __init__(self, num_groups: int, layers: int, row_bytes: int, ring: int, logical_capacity: int,
                 gpu_slots: int, host_slots: int, max_sets: int, max_k: int, max_append: int = 4096,
                 device: str = "cuda", stream=None, policy: int = 0, static_workspace: bool = False,
                 placement: int = 0):
        """policy: POLICY_PBLRU (0) or POLICY_LRU (1). static_workspace: take the device
        workspace from the library's static array (ula_init_static) instead of a torch
        allocation. placement: PLACE_LOWEST (0) or PLACE_RING (1) for appended entries."""
        import torch
        self.cfg = UlaConfig(num_groups, layers, row_bytes, ring, logical_capacity, gpu_slots,
                             host_slots, max_sets, max_k, max_append, policy, placement)
        self.policy = policy
        L = lib()
        nbytes = L.ula_device_bytes(ctypes.byref(self.cfg))
        if nbytes == 0:
            raise UlaError(-1, "ula_device_bytes", "invalid configuration")
        self.device_bytes = nbytes
        self.host_bytes = L.ula_host_bytes(ctypes.byref(self.cfg))
        self.ws = None if static_workspace else torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.host = None
        if self.host_bytes:
            self.host = L.ula_host_alloc(self.host_bytes)
            if not self.host:
                raise UlaError(-8, "ula_host_alloc", f"could not pin {self.host_bytes} bytes")
        self.ctx = ctypes.c_void_p()
        if static_workspace:
            rc = L.ula_init_static(ctypes.byref(self.cfg), self.host, _stream(stream), ctypes.byref(self.ctx))
            if rc:
                L.ula_host_free(self.host)
                self.host = None
            _check(rc, "ula_init_static")
        else:
            _check(L.ula_init(ctypes.byref(self.cfg), self.ws.data_ptr(), self.host, _stream(stream),
                              ctypes.byref(self.ctx)), "ula_init")
        self.num_groups, self.layers, self.row_bytes, self.ring = num_groups, layers, row_bytes, ring
        self.N, self.P, self.H = logical_capacity, gpu_slots, host_slots

    # -- calls ---------------------------------------------------------------
    def _rows(self, las, rows, what):
        """(pointer, on_device, keep) for the appended rows [n][layers][row_bytes];
        `keep` holds a host copy alive for the duration of the call."""
        n = las.size * self.layers * self.row_bytes
        if hasattr(rows, "is_cuda") and rows.is_cuda:
            return (_dev(rows, "uint8", n, what) if las.size else None), 1, None
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        if rows.size < n:
            raise ValueError(f"{what}: {rows.size} row bytes, at least {n} needed")
        return (rows.ctypes.data if las.size else None), 0, rows

    def append(self, group: int, las: np.ndarray, rows, stream=None) -> None:
        """rows: torch CUDA uint8 tensor or numpy uint8 array [n][layers][row_bytes]."""
        las = np.ascontiguousarray(las, dtype=np.int32)
        ptr, on_dev, _keep = self._rows(las, rows, "ula_append rows")
        _check(lib().ula_append(self.ctx, group, las.size, las.ctypes.data, ptr, on_dev,
                                _stream(stream)), "ula_append")

    def release(self, group: int, las: np.ndarray, stream=None) -> None:
        """Give back the slots of finished entries (they become absent)."""
        las = np.ascontiguousarray(las, dtype=np.int32)
        _check(lib().ula_release(self.ctx, group, las.size, las.ctypes.data, _stream(stream)),
               "ula_release")

    def step(self, group: int, sel, stream=None) -> None:
        """sel: torch CUDA int32 tensor [n_sets][k] (or [k] for one set)."""
        n_sets, k = _sets(sel)
        _check(lib().ula_step(self.ctx, group, n_sets, k, _dev(sel, "int32", n_sets * k, "ula_step sel"),
                              _stream(stream)), "ula_step")

    def append_step(self, group: int, las: np.ndarray, rows, sel, stream=None) -> None:
        """append(group, las, rows) then step(group, sel), in fewer launches."""
        las = np.ascontiguousarray(las, dtype=np.int32)
        ptr, on_dev, _keep = self._rows(las, rows, "ula_append_step rows")
        n_sets, k = _sets(sel)
        _check(lib().ula_append_step(self.ctx, group, las.size, las.ctypes.data if las.size else None,
                                     ptr, on_dev, n_sets, k,
                                     _dev(sel, "int32", n_sets * k, "ula_append_step sel"),
                                     _stream(stream)), "ula_append_step")

    def gather(self, group: int, layer: int, sel, out=None, stream=None):
        import torch
        n_sets, k = _sets(sel)
        if out is None:
            out = torch.empty((n_sets, k, self.row_bytes), dtype=torch.uint8, device=sel.device)
        _check(lib().ula_gather(self.ctx, group, layer, n_sets, k,
                                _dev(sel, "int32", n_sets * k, "ula_gather sel"),
                                _dev(out, "uint8", n_sets * k * self.row_bytes, "ula_gather out"),
                                _stream(stream)), "ula_gather")
        return out

    def gather_layers(self, group: int, layer0: int, n_layers: int, sel, out=None, stream=None):
        """Layers layer0 .. layer0 + n_layers - 1 in one launch: out[i] is gather(layer0 + i)."""
        import torch
        n_sets, k = _sets(sel)
        if out is None:
            out = torch.empty((max(n_layers, 0), n_sets, k, self.row_bytes), dtype=torch.uint8,
                              device=sel.device)
        _check(lib().ula_gather_layers(
            self.ctx, group, layer0, n_layers, n_sets, k,
            _dev(sel, "int32", n_sets * k, "ula_gather_layers sel"),
            _dev(out, "uint8", max(n_layers, 0) * n_sets * k * self.row_bytes, "ula_gather_layers out"),
            _stream(stream)), "ula_gather_layers")
        return out

    def sync(self, stream=None) -> List[tuple]:
        st = (UlaStepStats * self.num_groups)()
        _check(lib().ula_sync(self.ctx, _stream(stream), st), "ula_sync")
        return [s.as_tuple() for s in st]

    def sync_code(self, stream=None) -> int:
        """ula_sync's return code without raising (for error-path tests)."""
        return lib().ula_sync(self.ctx, _stream(stream), None)

    def export_state(self, group: int) -> dict:
        W = (self.P + 31) // 32
        out = dict(map=np.empty(self.N, np.uint32), gown=np.empty(self.P, np.int32),
                   hown=np.empty(max(self.H, 1), np.int32),
                   bitsets=np.empty((self.ring + 2, W), np.uint32))
        stamps = np.empty(self.P, np.int32) if self.policy == POLICY_LRU else None
        sh = UlaStateHost(out["map"].ctypes.data, out["gown"].ctypes.data, out["hown"].ctypes.data,
                          out["bitsets"].ctypes.data, 0, 0, UlaStepStats(),
                          stamps.ctypes.data if stamps is not None else None)
        _check(lib().ula_export_state(self.ctx, group, ctypes.byref(sh)), "ula_export_state")
        out["hown"] = out["hown"][: self.H]
        out["cur"] = int(sh.cur)
        out["flag"] = int(sh.flag)
        out["stats"] = sh.last.as_tuple()
        if stamps is not None:
            out["stamps"] = stamps
        return out

    def read_rows(self, group: int, las: np.ndarray) -> np.ndarray:
        las = np.ascontiguousarray(las, dtype=np.int32)
        out = np.empty((las.size, self.layers, self.row_bytes), dtype=np.uint8)
        _check(lib().ula_read_rows(self.ctx, group, las.size, las.ctypes.data, out.ctypes.data),
               "ula_read_rows")
        return out

    def flag_address(self, group: int) -> int:
        p = ctypes.c_void_p()
        _check(lib().ula_flag_address(self.ctx, group, ctypes.byref(p)), "ula_flag_address")
        return p.value

    TIMING_STEP = 1      # phase events of every step (read_timing)
    TIMING_GATHER = 2    # kernel time of every gather (read_gather_timing)
    TIMING_LINK = 4      # kernel time of every step's host-link launch (read_link_timing)

    def set_timing(self, flags) -> None:
        """flags: an OR of TIMING_STEP and TIMING_GATHER (True means TIMING_STEP)."""
        flags = self.TIMING_STEP if flags is True else int(flags)
        _check(lib().ula_set_timing(self.ctx, flags), "ula_set_timing")

    def read_timing(self, group: int) -> List[float]:
        ms = (ctypes.c_float * 3)()
        _check(lib().ula_read_timing(self.ctx, group, ms), "ula_read_timing")
        return list(ms)

    def read_gather_timing(self) -> tuple:
        """(summed gather kernel milliseconds, launches) since the last read."""
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib().ula_read_gather_timing(self.ctx, ctypes.byref(ms), ctypes.byref(n)),
               "ula_read_gather_timing")
        return ms.value, n.value

    def read_link_timing(self) -> tuple:
        """(summed host-link launch milliseconds, launches) since the last read."""
        ms, n = ctypes.c_double(), ctypes.c_int64()
        _check(lib().ula_read_link_timing(self.ctx, ctypes.byref(ms), ctypes.byref(n)),
               "ula_read_link_timing")
        return ms.value, n.value

    def close(self) -> None:
        if getattr(self, "ctx", None) is not None and self.ctx.value:
            import torch
            torch.cuda.synchronize()
            lib().ula_destroy(self.ctx)
            self.ctx = None
        if getattr(self, "host", None):
            lib().ula_host_free(self.host)
            self.host = None
        self.ws = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
