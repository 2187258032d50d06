"""Host logic of bench.py (no GPU): the source digest that gates the stored
HBM-traffic figure, the parsing of the committed counter summary, and the
single-GPU guard."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_digest_is_stable_and_tracks_every_source(tmp_path, monkeypatch):
    for name in bench.FWD_SOURCES:
        (tmp_path / name).write_text(f"// {name}\n")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    d0 = bench.source_digest()
    assert d0 == bench.source_digest()
    assert len(d0) == 16 and all(c in "0123456789abcdef" for c in d0)
    for name in bench.FWD_SOURCES:
        p = tmp_path / name
        old = p.read_text()
        p.write_text(old + " ")
        assert bench.source_digest() != d0, name
        p.write_text(old)
    assert bench.source_digest() == d0


def test_stored_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    digest = bench.source_digest()
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("k") is None  # no summary
    (tmp_path / "k_pmc.md").write_text(f"source_digest: {digest}\nhbm_bytes_per_launch: 12345\n")
    assert bench.stored_traffic("k") == 12345.0
    (tmp_path / "k_pmc.md").write_text("source_digest: 0000000000000000\nhbm_bytes_per_launch: 12345\n")
    assert bench.stored_traffic("k") is None  # counters of another kernel version
    (tmp_path / "k_pmc.md").write_text(f"source_digest: {digest}\n")
    assert bench.stored_traffic("k") is None  # no figure


@pytest.mark.parametrize("tag,algorithmic", [
    ("bwd_dkdv_16traj_B64", 2_587_295_744),   # Q, dO, K, V, row terms read; dK, dV written
    ("decode_bf16_P8192", 34_213_888),        # K, V once per KV head, Q read; O, LSE written
    ("decode_bf16_P1024", 4_853_760),
])
def test_committed_counter_summaries_parse(tag, algorithmic):
    text = open(os.path.join(bench.PROFILES, f"{tag}_pmc.md")).read()
    assert "FETCH_SIZE" in text and "WRITE_SIZE" in text and "source_digest:" in text
    t = bench.stored_traffic(tag)
    # None once the kernel has changed since the counters were taken
    assert t is None or t >= algorithmic


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
