"""Host-side logic of bench.py (no GPU needed): the counter-measured traffic
is reported only for the kernel source it was taken on, and the one-GPU
contract refuses other GPU counts."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary(path, digest, total="82795729"):
    with open(path, "w") as f:
        f.write("# header line: ignored\n")
        f.write("kernel: decode_fused_kernel<4, 4, 3, false, false>\n")
        f.write(f"hbm_bytes_per_launch: {total}\n")
        f.write(f"source_digest: {digest}\n")


def test_traffic_reported_only_for_matching_source(tmp_path, monkeypatch):
    p = tmp_path / "traffic.txt"
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(p))
    assert bench.measured_traffic() is None            # no summary
    _summary(p, bench.kernel_source_digest())
    assert bench.measured_traffic() == 82795729.0       # taken on these sources
    _summary(p, "0" * 16)
    assert bench.measured_traffic() is None            # sources changed since
    _summary(p, bench.kernel_source_digest(), total="n/a")
    assert bench.measured_traffic() is None            # unreadable figure


def test_source_digest_covers_every_fused_decode_source(tmp_path, monkeypatch):
    """Changing any of the files the fused decode is built from changes the
    digest (so stale counters are never reported)."""
    base = bench.kernel_source_digest()
    for rel in bench.TRAFFIC_SOURCES:
        root = tmp_path / rel.replace("/", "_")
        root.mkdir()
        for other in bench.TRAFFIC_SOURCES:
            dst = root / other
            dst.parent.mkdir(parents=True, exist_ok=True)
            data = open(os.path.join(ROOT, other), "rb").read()
            dst.write_bytes(data + (b"\n" if other == rel else b""))
        monkeypatch.setattr(bench, "ROOT", str(root))
        assert bench.kernel_source_digest() != base, rel
    monkeypatch.setattr(bench, "ROOT", ROOT)
    assert bench.kernel_source_digest() == base


def test_prefill_traffic_uses_its_own_sources_and_key(tmp_path):
    """The prefill summary is keyed on the prefill sources' digest, and the
    figure is looked up by name (table and note lines are not read)."""
    p = tmp_path / "pf.txt"
    dig = bench.kernel_source_digest(bench.PREFILL_SOURCES)
    assert dig != bench.kernel_source_digest()
    with open(p, "w") as f:
        f.write("| kernel | read: MB |\n- note: text\n")
        f.write(f"fc1_hbm_bytes_per_launch: 677620306\nsource_digest: {dig}\n")
    got = bench.measured_traffic(str(p), bench.PREFILL_SOURCES, "fc1_hbm_bytes_per_launch")
    assert got == 677620306.0
    assert bench.measured_traffic(str(p), None, "fc1_hbm_bytes_per_launch") is None
    assert bench.measured_traffic(str(p), bench.PREFILL_SOURCES, "fc2_hbm_bytes_per_launch") is None


def test_committed_summaries_parse():
    """Both committed counter summaries carry a digest and their figures."""
    for path, key in ((bench.TRAFFIC_SUMMARY, "hbm_bytes_per_launch"),
                      (bench.PREFILL_TRAFFIC_SUMMARY, "fc1_hbm_bytes_per_launch")):
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith(("#", "|", "-")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        assert len(kv["source_digest"]) == 16
        assert float(kv[key]) > 0


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
