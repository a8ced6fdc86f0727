"""Device-side row generator (libulasynth.so): fills torch CUDA buffers with the
same bytes as synth.rows.rows_for, for the GPU side of the tests and the bench."""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libulasynth.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with synth.build.build()")
        # torch ships its own HIP runtime under the same soname as the one this
        # library links; importing torch first makes the library bind to that
        # runtime (loaded the other way round, the process ends up with two HIP
        # runtimes and device calls fail)
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.ulasynth_fill_rows.restype = ctypes.c_int
        L.ulasynth_fill_rows.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_uint64]
        _lib = L
    return _lib


def fill_rows(out, las, layers: int, row_bytes: int, seed: int, group: int, stream=None):
    """out: CUDA uint8 tensor of n*layers*row_bytes bytes; las: CUDA int32 tensor [n]."""
    import torch
    s = torch.cuda.current_stream().cuda_stream if stream is None else stream.cuda_stream
    n = las.numel()
    assert out.numel() >= n * layers * row_bytes and out.is_cuda and las.is_cuda
    assert las.dtype == torch.int32 and las.is_contiguous() and out.is_contiguous()
    rc = lib().ulasynth_fill_rows(out.data_ptr(), las.data_ptr(), n, layers, row_bytes, seed, group, s)
    if rc != 0:
        raise RuntimeError(f"ulasynth_fill_rows failed ({rc})")
    return out


def rows_device(las_np, layers: int, row_bytes: int, seed: int, group: int):
    """Rows of the given addresses as a CUDA uint8 tensor [n][layers][row_bytes]."""
    import numpy as np
    import torch
    las = torch.from_numpy(np.ascontiguousarray(las_np, dtype=np.int32)).cuda()
    out = torch.empty((las.numel(), layers, row_bytes), dtype=torch.uint8, device="cuda")
    return fill_rows(out, las, layers, row_bytes, seed, group)
