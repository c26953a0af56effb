"""Host checks (no GPU) of how the library carves caller workspaces.

The top-k plan and its candidate areas are plain C++ (csrc/workspace.hpp); a small driver
compiled here with the host compiler sweeps plans and checks every area against the bytes the
C ABI asks for.  The library's own *_workspace_bytes answers are checked against the scores and
partial-output sizes the launchers carve."""
import ctypes
import os
import shutil
import subprocess

import pytest

from compressed_attention_long_amd import _lib as L

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "compressed_attention_long_amd", "csrc")


@pytest.mark.parametrize("sanitize", [False, True])
def test_workspace_carving_fits(tmp_path, sanitize):
    """The plan sweep, built plain and with the host compiler's address and undefined-behaviour
    sanitizers (host code only: the driver includes no device code)."""
    cxx = shutil.which("g++") or shutil.which("c++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = tmp_path / "carving"
    flags = ["-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"] if sanitize else []
    build = subprocess.run([cxx, "-std=c++17", "-O1", "-Wall", *flags, "-I", CSRC,
                            os.path.join(HERE, "host", "workspace_carving.cpp"), "-o", str(exe)],
                           capture_output=True, text=True)
    if sanitize and build.returncode != 0:
        pytest.skip("the host compiler cannot build with sanitizers here: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr[-4000:]
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout[-4000:]
    assert "0 failures" in r.stdout


def test_index_workspace_holds_scores_and_candidates():
    lib = L.load()
    for B, Tq, cap, k in [(32, 1, 16383, 1024), (4, 1, 262143, 1024), (4, 1, 524288, 512), (1, 4096, 33791, 1024),
                          (1, 1, 300000, 4096), (2, 3, 70000, 1)]:
        need = L.index_topk_workspace_bytes(B, Tq, 64, cap, k)
        scores = (B * Tq * cap * 4 + 255) // 256 * 256
        assert need >= scores and need % 256 == 0
