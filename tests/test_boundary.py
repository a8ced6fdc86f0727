"""The C-ABI library loads and exports every symbol include/ula.h declares.

No compute call is made here: only the pure host functions (sizes, error
texts) and configuration rejection, which return before touching a device.
"""

import ctypes
import os
import re

import pytest

from serving_pb_lru_amd import ula
from synth import Trace, preset

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "ula.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ula_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 16
    L = ula.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(n for n, _, _ in ula.SIGNATURES) == names


def test_synth_device_library_exports_filler():
    from synth import device
    assert hasattr(device.lib(), "ulasynth_fill_rows")


def test_probe_library_exports_and_rejects_bad_arguments():
    """bench.py's measurement probes: the row-move and copy entry points refuse
    bad arguments on the host, before any device call."""
    from measure import probes
    L = probes.lib()
    p = ctypes.c_void_p(16)
    assert L.probe_move_rows(3, p, p, p, 1, 656, 1, 0) == -1            # no such mode
    assert L.probe_move_rows(-1, p, p, p, 1, 656, 1, 0) == -1           # no such mode
    assert L.probe_move_rows(0, None, p, p, 1, 656, 1, 0) == -1         # null pointer
    assert L.probe_move_rows(0, p, p, p, 1, 650, 1, 0) == -1            # not 16-byte pieces
    assert L.probe_move_rows(1, p, p, p, 1, 656, 0, 0) == -1            # no workgroups
    assert L.probe_move_rows(0, p, p, p, 1 << 27, 656, 1, 0) == -1      # piece index past 32 bits
    assert L.probe_copy(None, p, 16, 1, 0, 0) == -1                          # null pointer
    assert L.probe_copy(p, p, 24, 1, 1, 0) == -1                             # not 16-byte pieces
    assert L.probe_copy(ctypes.c_void_p(8), p, 16, 1, 0, 0) == -1            # misaligned
    assert L.probe_copy(p, p, 16, 0, 1, 0) == -1                             # no workgroups
    assert L.probe_copy(p, p, 1 << 36, 1, 0, 0) == -1                        # piece index past 32 bits
    assert L.probe_copy(p, p, 0, 1, 1, 0) == 0                               # nothing to copy


def _cfg(**kw):
    base = dict(num_groups=1, layers_per_group=3, row_bytes=656, ring_buckets=8,
                logical_capacity=1049600, gpu_slots=524288, host_slots=525312, max_sets=16,
                max_k=2048, max_append=4096)
    base.update(kw)
    return ula.UlaConfig(**base)


def test_sizes_cover_pools():
    L = ula.lib()
    c = _cfg()
    dev = L.ula_device_bytes(ctypes.byref(c))
    host = L.ula_host_bytes(ctypes.byref(c))
    assert dev >= 524288 * 3 * 656 + 1049600 * 12
    assert host == 525312 * 3 * 656
    for name in ["tiny_4x4k", "evict_r256_128k_g2"]:
        tr = Trace(preset(name))
        wl = tr.wl
        c = _cfg(num_groups=wl.groups, layers_per_group=wl.layers, ring_buckets=wl.ring,
                 logical_capacity=tr.N, gpu_slots=tr.P, host_slots=tr.H, max_sets=tr.n_sets, max_k=tr.k)
        assert L.ula_device_bytes(ctypes.byref(c)) > tr.P * wl.layers * 656 * wl.groups
        assert L.ula_host_bytes(ctypes.byref(c)) == tr.H * wl.layers * 656 * wl.groups


@pytest.mark.parametrize("bad", [
    dict(row_bytes=650), dict(row_bytes=0), dict(ring_buckets=0), dict(ring_buckets=65),
    dict(gpu_slots=0), dict(host_slots=-1), dict(num_groups=0), dict(max_k=0),
    dict(logical_capacity=0), dict(gpu_slots=2 ** 31 - 10, host_slots=100),
    dict(max_sets=1 << 16, max_k=1 << 16), dict(policy=2), dict(policy=-1), dict(max_append=0),
    dict(layers_per_group=0), dict(layers_per_group=257), dict(row_bytes=4112),
    dict(placement=2), dict(placement=-1), dict(placement=1, policy=1)])
def test_bad_configs_rejected_on_host(bad):
    L = ula.lib()
    c = _cfg(**bad)
    assert L.ula_device_bytes(ctypes.byref(c)) == 0
    assert L.ula_host_bytes(ctypes.byref(c)) == 0
    ctx = ctypes.c_void_p()
    assert L.ula_init(ctypes.byref(c), None, None, 0, ctypes.byref(ctx)) == -1
    assert not ctx.value


def test_error_texts():
    L = ula.lib()
    for code, name in ula.ERROR_NAMES.items():
        assert L.ula_strerror(code)
    assert L.ula_strerror(-5).decode().startswith("a step selects more distinct")
    assert L.ula_destroy(None) == -1


def test_binding_rejects_unusable_device_buffers():
    """The binding passes plain pointers, so it checks every device buffer before a
    call: a CUDA tensor of the right dtype, contiguous, and large enough for what
    the call reads or writes."""
    import torch

    class FakeCuda:   # stands in for a CUDA tensor (no GPU here)
        is_cuda = True

        def __init__(self, dtype, n, contiguous=True):
            self.dtype, self.n, self.contiguous = dtype, n, contiguous

        def is_contiguous(self):
            return self.contiguous

        def numel(self):
            return self.n

        def data_ptr(self):
            return 4096

    assert ula._dev(FakeCuda(torch.int32, 8), "int32", 8, "sel") == 4096
    assert ula._dev(FakeCuda(torch.uint8, 0), "uint8", 0, "out") == 4096
    bad = [torch.zeros(8, dtype=torch.int32),            # host memory
           FakeCuda(torch.int64, 8),                     # wrong dtype
           FakeCuda(torch.int32, 7),                     # too small
           FakeCuda(torch.int32, 8, contiguous=False)]   # strided view
    for t in bad:
        with pytest.raises(ValueError):
            ula._dev(t, "int32", 8, "sel")


def test_static_workspace_refuses_a_large_config_on_host():
    """ula_init_static checks the configuration against its static workspace (32 MiB)
    before it touches a device."""
    L = ula.lib()
    c = _cfg()   # about 1.1 GB of workspace
    ctx = ctypes.c_void_p()
    assert L.ula_init_static(ctypes.byref(c), None, 0, ctypes.byref(ctx)) == -10
    assert not ctx.value
    assert L.ula_strerror(-10).decode().startswith("the configuration needs more device workspace")
    bad = _cfg(row_bytes=650)
    assert L.ula_init_static(ctypes.byref(bad), None, 0, ctypes.byref(ctx)) == -1
