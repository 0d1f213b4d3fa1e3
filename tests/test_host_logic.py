"""Host-side logic, on the CPU: the visibility intervals and tile predicates
that set every kernel's loop ranges and masking, checked against a brute-force
enumeration, and the first row of every tile load of every kernel, checked to
lie inside its tensor for every geometry the kernels accept (the short-
sequence backward: every Nk <= 224 and Nq <= 1024 under every mask)
(tests/host/tile_range_check.cpp, built with g++ and the address and
undefined-behaviour sanitizers)."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_tile_ranges_against_brute_force(tmp_path):
    exe = tmp_path / "tile_range_check"
    cmd = ["g++", "-std=c++17", "-O1", "-Wall", "-Werror", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-I", os.path.join(ROOT, "head_attention_attn_amd", "csrc"),
           os.path.join(HERE, "host", "tile_range_check.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("0 failures")


def test_attention_module_rejects_unknown_mask():
    import pytest
    import head_attention_attn_amd as attn
    with pytest.raises(ValueError):
        attn.FusedAttention(mask="diagonal")
    assert "causal" in repr(attn.FusedAttention(mask="causal"))
