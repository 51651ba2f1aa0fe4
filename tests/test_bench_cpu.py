"""CPU: bench.py's host logic. It refuses more than one GPU, and it reads the committed
rocprofv3 traffic records: scaled counter bytes, or None once a listed kernel source has
changed since the counters were taken."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def _tree(tmp_path, src_text: str):
    """A minimal tree: one kernel source under the package's csrc/ and a profiles/ folder."""
    csrc = tmp_path / "mixture_experts_ffn_ids_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "k.hip").write_text(src_text)
    (tmp_path / "profiles").mkdir()
    return tmp_path


def test_traffic_record_is_scaled_and_tied_to_the_sources(tmp_path, monkeypatch):
    root = _tree(tmp_path, "kernel v1\n")
    monkeypatch.setattr(bench, "ROOT", str(root))
    sha = bench.source_sha256(["k.hip"])
    (root / "profiles" / "gate_up_w.md").write_text(
        "# summary\n\ntraffic-record: kernel=gate_up workload=w fetch_kib=100.0 write_kib=10.0 "
        f"fetch_scale=2.0 write_scale=1.0 sources=k.hip source_sha256={sha}\n")
    assert bench.stored_traffic("w") == (100 * 2 + 10) * 1024
    assert bench.stored_traffic("missing") is None
    # the kernel changes after the counters were taken: the record no longer applies
    (root / "mixture_experts_ffn_ids_amd" / "csrc" / "k.hip").write_text("kernel v2\n")
    assert bench.stored_traffic("w") is None


def test_committed_profiles_carry_well_formed_records():
    names = [n for n in os.listdir(os.path.join(ROOT, "profiles")) if n.startswith("gate_up_") and n.endswith(".md")]
    assert names, "no committed profile summaries"
    for n in names:
        text = open(os.path.join(ROOT, "profiles", n)).read()
        recs = [ln for ln in text.splitlines() if ln.startswith("traffic-record:")]
        assert len(recs) == 1, n
        rec = dict(kv.split("=", 1) for kv in recs[0].split()[1:])
        assert rec["kernel"] == "gate_up" and f"gate_up_{rec['workload']}.md" == n
        for k in ("fetch_kib", "write_kib", "fetch_scale", "write_scale"):
            assert float(rec[k]) > 0, (n, k)
        assert re.fullmatch(r"[0-9a-f]{64}", rec["source_sha256"]), n
        for src in rec["sources"].split(","):
            assert os.path.exists(os.path.join(ROOT, "mixture_experts_ffn_ids_amd", "csrc", src)), (n, src)
        # each summary gives the commands that produced it
        assert "rocprofv3 --kernel-trace --stats" in text and "rocprofv3 --pmc FETCH_SIZE" in text, n
