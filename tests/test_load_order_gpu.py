"""Regression: the binding loads libula.so (and the synthetic-row and probe
libraries) only after torch, so that they bind to torch's HIP runtime. Loaded
the other way round, a process held two HIP runtimes and every later device call
failed. The check runs in a child process, which loads libula.so before anything
else touches torch."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys
sys.path.insert(0, {root!r})
import serving_pb_lru_amd.ula as u
u.lib()                                   # before torch has been imported here
import numpy as np
import torch
from synth import Trace, preset, rows_for
from synth.device import rows_device
from serving_pb_lru_amd.replay import engine_for
torch.cuda.set_device(0)
tr = Trace(preset("tiny_4x4k"), steps=1)
wl = tr.wl
eng = engine_for(tr)
las = tr.initial_load_order()
eng.append(0, las, rows_device(las, wl.layers, wl.row_bytes, wl.seed, 0))
app = tr.appends(1)
sel = next(tr.selections(0))
eng.append_step(0, app, rows_for(wl.seed, 0, app, wl.layers, wl.row_bytes), torch.from_numpy(sel).cuda())
out = eng.gather(0, 0, torch.from_numpy(sel).cuda()).cpu().numpy()
eng.sync()
flat = sel.reshape(-1)
want = np.zeros((flat.size, wl.row_bytes), np.uint8)
ok = flat >= 0
want[ok] = rows_for(wl.seed, 0, flat[ok], wl.layers, wl.row_bytes)[:, 0]
assert np.array_equal(out.reshape(want.shape), want)
eng.close()
print("load order ok", flush=True)
"""


def test_library_loaded_before_torch():
    r = subprocess.run([sys.executable, "-c", CHILD.format(root=ROOT)], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0 and "load order ok" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
