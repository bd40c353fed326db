"""The table-driven kernels' symbol classification (ppr_slots.h) on the host.

The slot tables and the four-byte classification are built here with g++ and
v_perm_b32 emulated from its instruction-set definition. For the workloads'
delimiter sets and 3000 random sets of up to 8 special bytes anywhere in
0..255, every byte value at every position of a word must get its class code;
a table whose slot function is blind to the one false-match difference must
fail, which shows the check sees that case.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "dfa_parsing_delimiter_amd", "csrc")


def test_every_byte_classified(tmp_path):
    exe = str(tmp_path / "slots_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-Wall", "-I", CSRC, "-o", exe,
                    os.path.join(HERE, "host", "slots_check.cpp")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "slots ok" in r.stdout
