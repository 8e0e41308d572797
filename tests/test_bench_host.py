"""Host-side logic of bench.py, no GPU: the one-GPU refusal, the key that ties a counter summary to
the kernel source it was taken on, and the visible-pair count behind the step-1 flop figure."""
import os
import subprocess
import sys

import numpy as np
import pytest

import qi_inputs as qin
from oracle import qi_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    # the refusal comes before anything touches the GPU (torch is not even imported)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SRC).read()
    h = bench.kernel_hash()
    commented = tmp_path / "commented.hip"
    commented.write_text("// a new comment line\n\n" + src.replace("\n", "  // trailing\n", 3) + "\n\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(commented))
    assert bench.kernel_hash() == h
    changed = tmp_path / "changed.hip"
    changed.write_text(src + "\nstatic int one_more_line;\n")
    monkeypatch.setattr(bench, "KERNEL_SRC", str(changed))
    assert bench.kernel_hash() != h


def test_counter_summary_used_only_for_its_own_kernel(tmp_path, monkeypatch):
    prof = tmp_path / "counters.md"
    prof.write_text(f"kernel_source_sha256_16: {bench.kernel_hash()}\nhbm_bytes_per_launch: 392709001\n"
                    "sclk_median_ghz: 1.931\n")
    monkeypatch.setattr(bench, "PROFILE", str(prof))
    assert bench.traffic_from_profile() == 392709001.0
    assert bench.sclk_from_profile() == pytest.approx(1.931)
    prof.write_text("kernel_source_sha256_16: 0123456789abcdef\nhbm_bytes_per_launch: 392709001\n"
                    "sclk_median_ghz: 1.931\n")
    assert bench.traffic_from_profile() is None
    assert bench.sclk_from_profile() is None
    monkeypatch.setattr(bench, "PROFILE", str(tmp_path / "missing.md"))
    assert bench.traffic_from_profile() is None


@pytest.mark.parametrize("name", ["tiny_f32", "txt256_ref32_tgt32", "txt512_tgt64", "txt512_10ref32_tgt64",
                                  "interleaved10"])
def test_visible_pairs_equal_the_oracle_mask(name):
    segs = {**qin.WORKLOADS, **qin.INTERLEAVED_WORKLOADS}[name].segments
    S = sum(s.n_tokens for s in segs)
    if S <= 6000:
        want = int(O.mask_dense(segs).sum())
    else:   # rows in blocks, to bound memory
        want = sum(int(O.mask_rows(segs, np.arange(r, min(r + 2048, S))).sum()) for r in range(0, S, 2048))
    assert bench.visible_pairs_per_head(segs) == want


def test_visible_pairs_headline():
    # 273.2 M visible (query, key) pairs per head at step 1 of the 21,504-token layout: 3.3565 TFLOP
    # over 24 heads at 4 * 128 flops per pair
    segs = qin.WORKLOADS["txt1024_4ref64_tgt64"].segments
    n = bench.visible_pairs_per_head(segs)
    assert n == O.visible_pairs(segs)
    assert round(n / 1e6, 1) == 273.2
    assert round(4 * 128 * 24 * n / 1e12, 4) == 3.3565
