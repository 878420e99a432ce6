"""Host-side checks of bench.py's contract (no GPU).

* one GPU only: --gpus above 1 exits with a message before touching a device;
* the algorithmic byte counts per token and KV head that the roofline divides
  by are the closed profiles' payloads (Paged KV Context Store page, X-extent
  list; the benchmark configurations name fp32 scale planes): BF16 D=128 is
  two 256-byte code rows, INT8-G64 D=128 two 128-byte code rows and two
  fp32 scales per side, K8V4 D=256 a 256-byte FP8 row plus one fp32 scale
  (K) and a 128-byte E2M1 row plus sixteen E4M3 scale bytes (V);
* the append happens inside the decode run only where every entry appends
  one row (the run writes one row per entry);
* the committed HBM traffic summaries parse, name their kernel and source
  hash, and stay within a few percent above the algorithmic bytes they were
  measured against (traffic well above them would mean re-reads).  The bound
  holds for the bandwidth-bound launches (64 MB and more).  A tiny launch
  (one 300-token entry, 314 KB) is only held to reading at least its
  algorithmic bytes: its raw fetch counter reads 1.06x those bytes, but the
  copy calibration (taken over 1 GiB, counter factor 0.5) doubles that, so
  the calibrated figure does not carry to a launch that small.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


@pytest.mark.parametrize("profile,D,sb,want", [
    ("BF16", 128, 4, 2 * 128 * 2),
    ("INT8_G64", 128, 4, 2 * (128 + 2 * 4)),
    ("INT8_G64", 128, 2, 2 * (128 + 2 * 2)),
    ("K8V4", 256, 4, (256 + 4) + (128 + 16)),
])
def test_roofline_bytes_per_token_and_head(profile, D, sb, want):
    import bench
    assert bench.bytes_per_token_head(profile, D, sb) == want


def _summaries():
    d = os.path.join(ROOT, "profiles")
    return sorted(os.path.join(d, f) for f in os.listdir(d) if "_traffic_" in f)


@pytest.mark.parametrize("path", _summaries(), ids=os.path.basename)
def test_traffic_summaries_are_consistent(path):
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    assert kv.get("kernel")
    assert len(kv.get("source_sha256", "")) == 64
    traffic = float(kv["traffic_bytes_per_dispatch"])
    alg = float(kv.get("algorithmic_bytes_per_dispatch") or kv["algorithmic_kv_bytes_per_dispatch"])
    if "call_traffic_bytes" in kv:
        traffic = float(kv["call_traffic_bytes"])
    assert alg > 0
    assert traffic >= 0.95 * alg, (traffic, alg)
    if alg >= 64e6:
        assert traffic <= 1.10 * alg, (traffic, alg)


def test_append_inside_the_run_only_for_one_row_per_entry():
    # paged_attn_decode_append_run writes one row per entry at seq_len - 1:
    # the step may stand on it only where every entry appends one row
    import bench
    import workloads
    assert bench.step_append_fused(workloads.get(2))
    assert bench.step_append_fused(workloads.get(4))
    wl3 = workloads.get(3)
    assert sum(wl3.step) > wl3.B
    assert not bench.step_append_fused(wl3)
