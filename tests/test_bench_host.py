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


def _point_at(monkeypatch, tmp_path, workload):
    """Make bench read workload's summary from tmp_path (same sources)."""
    name, sources = bench.TRAFFIC[workload]
    table = dict(bench.TRAFFIC)
    table[workload] = (os.path.join(str(tmp_path), name), sources)
    monkeypatch.setattr(bench, "TRAFFIC", table)
    return tmp_path / name, sources


def test_traffic_reported_only_for_matching_source(tmp_path, monkeypatch):
    p, sources = _point_at(monkeypatch, tmp_path, "decode4")
    assert bench.measured_traffic("decode4") is None            # no summary
    _summary(p, bench.kernel_source_digest(sources))
    assert bench.measured_traffic("decode4") == 82795729.0       # taken on these sources
    _summary(p, "0" * 16)
    assert bench.measured_traffic("decode4") is None            # sources changed since
    _summary(p, bench.kernel_source_digest(sources), total="n/a")
    assert bench.measured_traffic("decode4") is None            # unreadable figure


def test_source_digest_covers_every_source_of_each_summary(tmp_path, monkeypatch):
    """Changing any of the files a summarized kernel is built from changes
    that summary's digest (so stale counters are never reported)."""
    for workload, (_, sources) in bench.TRAFFIC.items():
        base = bench.kernel_source_digest(sources)
        for rel in sources:
            root = tmp_path / workload / rel.replace("/", "_")
            root.mkdir(parents=True)
            for other in sources:
                dst = root / other
                dst.parent.mkdir(parents=True, exist_ok=True)
                data = open(os.path.join(ROOT, other), "rb").read()
                dst.write_bytes(data + (b"\n" if other == rel else b""))
            monkeypatch.setattr(bench, "ROOT", str(root))
            assert bench.kernel_source_digest(sources) != base, (workload, rel)
        monkeypatch.setattr(bench, "ROOT", ROOT)
        assert bench.kernel_source_digest(sources) == base


def test_prefill_traffic_uses_its_own_sources_and_key(tmp_path, monkeypatch):
    """The prefill summary is keyed on the prefill sources' digest, and the
    figure is looked up by name (table and note lines are not read)."""
    p, sources = _point_at(monkeypatch, tmp_path, "prefill")
    dig = bench.kernel_source_digest(sources)
    assert dig != bench.kernel_source_digest(bench.TRAFFIC_SOURCES)
    with open(p, "w") as f:
        f.write("| kernel | read: MB |\n- note: text\n")
        f.write(f"fc1_hbm_bytes_per_launch: 677620306\nsource_digest: {dig}\n")
    assert bench.measured_traffic("prefill", "fc1_hbm_bytes_per_launch") == 677620306.0
    assert bench.measured_traffic("prefill", "fc2_hbm_bytes_per_launch") is None
    with open(p, "w") as f:
        f.write(f"fc1_hbm_bytes_per_launch: 677620306\nsource_digest: "
                f"{bench.kernel_source_digest(bench.TRAFFIC_SOURCES)}\n")
    assert bench.measured_traffic("prefill", "fc1_hbm_bytes_per_launch") is None


def test_committed_summaries_parse():
    """Every committed counter summary carries a digest and its figure."""
    keys = {"prefill": "fc1_hbm_bytes_per_launch", "small32": "fc1_hbm_bytes_per_launch"}
    for workload, (name, _) in bench.TRAFFIC.items():
        path = os.path.join(ROOT, "profiles", name)
        if not os.path.exists(path):
            continue
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith(("#", "|", "-")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
        assert len(kv["source_digest"]) == 16, name
        assert float(kv[keys.get(workload, "hbm_bytes_per_launch")]) > 0, name


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
