"""Host-side logic of bench.py, no GPU: the reader of the committed HBM
counter summary and its kernel-source guard, the algorithmic byte count of a
layer call (checked by hand on a tiny layer), and the refusal of more than
one GPU."""
import os
import re
import subprocess
import sys
import types

import numpy as np

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_counted_traffic_reads_the_committed_summary():
    text = open(bench.PMC_SUMMARY).read()
    val = int(re.search(r"traffic_bytes_per_call:\s*([0-9]+)", text).group(1))
    sha = re.search(r"kernel_sources_sha256:\s*([0-9a-f]{64})", text).group(1)
    got = bench.counted_traffic()
    # the counted bytes are used only while the kernel sources are the ones counted
    assert got == (val if sha == bench.kernel_sources_sha() else None)
    if got is not None:
        # fetches of about the algorithmic 41.9 MB, plus the partial-row round trip
        assert 41_000_000 < got < 60_000_000


def test_counted_traffic_guard(tmp_path, monkeypatch):
    p = tmp_path / "pmc.md"
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(p))
    p.write_text("traffic_bytes_per_call: 123\nkernel_sources_sha256: " + "0" * 64 + "\n")
    assert bench.counted_traffic() is None                  # other sources
    p.write_text("traffic_bytes_per_call: 123\nkernel_sources_sha256: " +
                 bench.kernel_sources_sha() + "\n")
    assert bench.counted_traffic() == 123
    p.write_text("kernel_sources_sha256: " + bench.kernel_sources_sha() + "\n")
    assert bench.counted_traffic() is None                  # no traffic line
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.counted_traffic() is None


def test_layer_bytes_by_hand():
    """3 routed experts (top-2) and 1 shared, d = 128, f = 64, two tokens."""
    d, f = 128, 64
    L = types.SimpleNamespace(d=d, f=f, E=3, S=1, k=2)
    idx = np.array([[0, 2], [2, 1]])               # token 0: experts 0, 2; token 1: 2, 1
    masks = np.zeros((2, 3, f), np.uint8)
    masks[0, 0, :10] = 1                           # expert 0: channels 0-9
    masks[0, 1, 5:20] = 1                          # expert 2, token 0: 5-19
    masks[1, 0, 15:30] = 1                         # expert 2, token 1: 15-29 (union 5-29: 25)
    masks[1, 1, :3] = 1                            # expert 1: 0-2
    masks[0, 2, :8] = 1                            # shared, token 0: 0-7
    masks[1, 2, 4:12] = 1                          # shared, token 1: 4-11 (union 0-11: 12)
    io = 3 * d * 2 + 2 * d * 2 + 2 * d * 4         # router rows, x in (16-bit), y out (fp32)
    codes = d * f // 4 + 4 * f * (d // 64)         # INT2 codes and group scales of one expert
    rows = lambda n: 2 * n * d * 2                 # gate and down rows of n channels
    want = io + (codes + rows(10)) + (codes + rows(3)) + (codes + rows(25)) + (codes + rows(12))
    assert bench.layer_bytes(L, masks, idx) == want
    # experts 2 and the shared one on the dense path read three 16-bit matrices each
    dense = np.array([0, 0, 1, 1], np.uint8)
    want_d = io + (codes + rows(10)) + (codes + rows(3)) + 2 * (3 * d * f * 2)
    assert bench.layer_bytes(L, masks, idx, dense) == want_d
    # an expert that no token chose costs nothing, even if its mask slot holds ones
    idx1 = np.array([[0, 1], [1, 0]])
    want1 = io + (codes + rows(len(set(range(10)) | set(range(3))))) + \
        (codes + rows(len(set(range(5, 20)) | set(range(15, 30))))) + (codes + rows(12))
    assert bench.layer_bytes(L, masks, idx1) == want1


def test_more_than_one_gpu_is_refused():
    env = dict(os.environ)
    env.pop("WORLD_SIZE", None)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 2, r.stderr
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""                  # no JSON line
