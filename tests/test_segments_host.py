"""The decode's segmentation arithmetic checked on the host, over random batches.

The kernels take their segment length, merge ranges and partial-record slots from
csrc/segments.hpp; tests/native/segments_driver.cpp compiles that header for the host and
checks, for random lengths, head groupings, partition sizes and grid sizes (with the
host's bound on the lengths sometimes below the longest length on the device):
  * every work unit lies in exactly one segment below the grid size W;
  * each wave's search finds the text and unit where its segment starts;
  * each run's merge range is exactly the segments it touches, never past W - 1;
  * no two runs write the same partial record and every record lies in the workspace.
The same driver with the segment length fixed to the partition length (the arithmetic
before a device length beyond the host's bound lengthened the segments) must fail.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_cache_320_amd", "csrc")
SRC = os.path.join(os.path.dirname(__file__), "native", "segments_driver.cpp")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(cc):
        pytest.skip("hipcc not available")
    exe = str(tmp_path_factory.mktemp("seg") / "segments_driver")
    subprocess.run([cc, "-O2", "-std=c++17", "-I", CSRC, SRC, "-o", exe], check=True,
                   capture_output=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_segmentation_covers_every_unit(driver, seed):
    r = subprocess.run([driver, str(seed), "1000"], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout + r.stderr


def test_fixed_segment_length_is_caught(driver):
    """With the segment length fixed to the partition length, a context longer than the
    host's bound leaves units to no wave: the check must say so."""
    r = subprocess.run([driver, "1", "1000", "old"], capture_output=True, text=True)
    assert r.returncode == 1 and "segments cover" in r.stdout, r.stdout + r.stderr
