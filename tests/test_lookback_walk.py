"""The decoupled look-back's walk over predecessors ends on every input.

The walk (dfa_parsing_delimiter_amd/csrc/ppr_walk.h, used by every single-pass
kernel) is built here for the host with g++ and run against a stub round that
never meets an inclusive prefix, the case after a look-back's bounded wait gives
up: the walk must end once tile 0 is covered, covering each predecessor once.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "dfa_parsing_delimiter_amd", "csrc")


def test_walk_terminates(tmp_path):
    exe = str(tmp_path / "walk_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-I", CSRC, "-o", exe,
                    os.path.join(HERE, "host", "walk_check.cpp")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "walk ok" in r.stdout
