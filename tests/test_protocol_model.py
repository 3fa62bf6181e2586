"""CPU model of the cross-workgroup exchange in the single-read acceptance kernel (tests/models/
acceptance_protocol.cpp): built with the host compiler and run over seeded trials of shapes, residency (all
chunks resident, fewer slots than a row's chunks, half) and wait limits (generous, short, zero). It checks that
every call returns, that alpha equals a single-threaded evaluation of the same arithmetic bit for bit, that the
workspace's sync region is zero after every call, and that nothing stops waiting when every chunk is resident."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs the host C++ compiler")
def test_acceptance_protocol_model(tmp_path):
    exe = tmp_path / "acceptance_protocol"
    src = os.path.join(HERE, "models", "acceptance_protocol.cpp")
    subprocess.run(["g++", "-O2", "-std=c++17", "-pthread", "-o", str(exe), src], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
