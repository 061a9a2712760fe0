"""Host-side parts of bench.py that need no GPU: the algorithmic byte and flop
counts behind the roofline fractions, the committed PMC traffic lookup, and the
one-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from ragged_attention_token_amd import workloads as wl  # noqa: E402


def test_algorithmic_bytes_of_the_headline_launches():
    """DeiT-S, B = 256, 40 kept per image (T = 10240), C = 384, bf16 in and out,
    worked out by hand from the per-unit figures:
      pack:   B N keep bytes + T (read + write a 3C row of 2-byte elements + a
              4-byte gather entry) + 4 (B + 1) offsets
            = 50432 + 10240 * (2 * 2304 + 4) + 1028 = 47278340
      attn:   T (3C in + C out, 2 bytes each) = 10240 * 3072 = 31457280
      unpack: T (read + write a C row + a gather entry) + offsets
            = 10240 * (2 * 768 + 4) + 1028 = 15770628
      flops:  4 L^2 d H per image = 256 * 4 * 1600 * 64 * 6 = 629145600."""
    w = wl.deits(256, 800)
    a = bench.algorithmic(w, 2)
    assert w.T == 10240
    assert a["pack"] == 47278340
    assert a["attn"] == 31457280
    assert a["unpack"] == 15770628
    assert a["attn_flops"] == 629145600
    # padded: every one of the B N positions, whatever the prune rate
    assert a["padded"] == 50432 * 3072 + 50432
    assert a["padded_flops"] == 4 * 256 * 197 * 197 * 64 * 6


def test_committed_traffic_is_read_only_for_the_current_source(tmp_path, monkeypatch):
    wl_name = "deits_b256_n197_h6_p800"
    got = bench.read_traffic("pack", wl_name)
    assert got is not None
    alg = bench.algorithmic(wl.deits(256, 800), 2)["pack"]
    assert abs(got / alg - 1.0) < 0.05  # measured HBM bytes near the algorithmic ones
    # a summary taken on another version of the source is ignored
    src = open(os.path.join(ROOT, "profiles", "pmc_pack_%s.txt" % wl_name)).read()
    lines = [("source_sha256: 0000000000000000" if l.startswith("source_sha256:") else l)
             for l in src.splitlines()]
    (tmp_path / ("pmc_pack_%s.txt" % wl_name)).write_text("\n".join(lines) + "\n")
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.read_traffic("pack", wl_name) is None
    assert bench.read_traffic("attn", wl_name) is None  # no summary at all


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
