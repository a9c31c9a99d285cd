"""Host-side checks of bench.py (no GPU): its one-GPU contract, the VALU issue roofline arithmetic,
and that every committed kernel profile under profiles/ was taken from the current kernel sources
(bench.py hashes the sources a profile covers into the profile, and reads its traffic back only
while the hash matches)."""
from __future__ import annotations

import glob
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 2
    assert "one GPU" in (r.stdout + r.stderr)


def test_valu_roofline_arithmetic():
    # 2.4e9 CU-clocks of plain instructions plus 1.2e9 transcendentals at two clocks each, over 256 CUs
    # at 2.4 GHz: 4.8e9 / 256 / 2.4 = 7.8125e6 ns
    vr = bench.valu_roofline(3.6e9, 1.2e9, 1.0e7)
    assert vr["bound_ns"] == pytest.approx(7.8125e6)
    assert vr["frac"] == pytest.approx(0.78125)


def _profile_hashes():
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        name = os.path.basename(path)
        m = re.search(r"^(?:kernel_)?source_sha256_16: (\S+)", open(path).read(), re.M)
        if name.startswith("engine_clock__"):
            continue   # clock readings carry no source hash
        yield name, (m.group(1) if m else None)


@pytest.mark.parametrize("name,recorded", list(_profile_hashes()))
def test_profiles_match_current_sources(name, recorded):
    assert recorded is not None, f"{name} records no source hash"
    workload = name.split("__", 1)[1][:-len(".txt")]
    if name.startswith("ce_split__"):
        current = bench.split_source_hash()
    else:
        current = bench.kernel_source_hash(workload)
    assert recorded == current, f"{name} was taken from other kernel sources: collect it again"
