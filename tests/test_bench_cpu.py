"""Host-side checks of bench.py that need no GPU: the one-GPU refusal of
--gpus N > 1, and the rotation size that keeps activation reads cold."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_rotation_exceeds_twice_the_infinity_cache():
    for nbytes in (1, 2 ** 20, 84 * 10 ** 6, 512 * 2 ** 20, 600 * 2 ** 20):
        n = bench._rotation(nbytes)
        assert n * nbytes >= 512 * 2 ** 20
        assert (n - 1) * nbytes < 512 * 2 ** 20 or n == 1


def test_sf_size_matches_padded_layout():
    # 128-row by 4-block tiles of the swizzled scale layout
    assert bench.sf_size(1, 16) == 128 * 4
    assert bench.sf_size(128, 64) == 128 * 4
    assert bench.sf_size(129, 80) == 256 * 8
    assert bench.sf_size(8192, 5120) == 8192 * 320
