"""include/ula.h is a C header: a C program that includes it compiles with gcc in
C11 mode, links against libula.so and calls the host-only entry points (the size
functions and the error texts, which touch no device), agreeing with the Python
binding. No GPU is needed."""

import ctypes
import os
import shutil
import subprocess

import pytest

from serving_pb_lru_amd import ula

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROGRAM = r"""
#include <stdio.h>
#include "ula.h"

int main(void) {
  ula_config c = {0};
  c.num_groups = 2; c.layers_per_group = 3; c.row_bytes = 656; c.ring_buckets = 8;
  c.logical_capacity = 100000; c.gpu_slots = 40000; c.host_slots = 60000;
  c.max_sets = 4; c.max_k = 2048; c.max_append = 4096;
  c.policy = ULA_POLICY_PBLRU; c.placement = ULA_PLACE_LOWEST;
  ula_config bad = c;
  bad.row_bytes = 650;                      /* not a multiple of 16 */
  printf("%zu %zu %zu\n", ula_device_bytes(&c), ula_host_bytes(&c), ula_device_bytes(&bad));
  printf("%s\n", ula_strerror(ULA_ECAPACITY));
  return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_header_compiles_as_c_and_links(tmp_path):
    lib_dir = os.path.dirname(ula.LIB_PATH)
    src = tmp_path / "use_ula.c"
    exe = tmp_path / "use_ula"
    src.write_text(PROGRAM)
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-L", lib_dir, "-lula", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    if r.returncode != 0 and "cannot find -lula" in r.stderr:
        # the library is named libula.so in-tree: link it by path instead
        r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                            ula.LIB_PATH, f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                           capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    dev, host, bad = (int(x) for x in out.stdout.split("\n")[0].split())
    cfg = ula.UlaConfig(2, 3, 656, 8, 100000, 40000, 60000, 4, 2048, 4096, 0, 0)
    L = ula.lib()
    assert dev == L.ula_device_bytes(ctypes.byref(cfg)) > 0
    assert host == L.ula_host_bytes(ctypes.byref(cfg)) == 2 * 60000 * 3 * 656
    assert bad == 0
    assert out.stdout.split("\n")[1] == L.ula_strerror(-5).decode()   # ULA_ECAPACITY
