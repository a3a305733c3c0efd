"""Host-side logic of bench.py (CPU only): the one-GPU guard and the lookup of
the committed HBM-traffic summaries, which must go stale when a kernel's
sources change."""
import importlib.util
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_committed_traffic_summaries_name_existing_sources():
    """Each committed summary lists the sources whose hash keys it, all of
    which exist, and its byte counts are positive."""
    for workload, kernels in (("attn_fwd_b2h16n8192d128", ("attn_fwd_bf16",)),
                              ("attn_fwd_b4h16n8192d128", ("attn_fwd_fp8", "blockquant_hadamard"))):
        with open(os.path.join(ROOT, "profiles", f"{workload}_traffic.json")) as f:
            rec = json.load(f)
        for kernel in kernels:
            k = rec["kernels"][kernel]
            assert k["sources"] and all(os.path.exists(os.path.join(ROOT, s)) for s in k["sources"])
            assert len(k["sha256"]) == 64 and k["read_bytes"] > 0 and k["write_bytes"] > 0


def test_traffic_lookup_follows_the_source_hash(tmp_path):
    """A summary counts only while the sources hash to its sha256: the lookup
    returns its bytes for an exact copy and None after any edit, or for an
    unknown kernel or workload."""
    import hashlib
    b = _bench()
    srcs = ["exact_attention_74_amd/csrc/attn_bf16.hip", "exact_attention_74_amd/csrc/common.h"]
    h = hashlib.sha256()
    for src in srcs:
        dst = tmp_path / src
        dst.parent.mkdir(parents=True, exist_ok=True)
        shutil.copy(os.path.join(ROOT, src), dst)
        h.update(dst.read_bytes())
    (tmp_path / "profiles").mkdir()
    rec = {"workload": "w", "kernels": {"k": {"sources": srcs, "sha256": h.hexdigest(),
                                              "read_bytes": 1000.0, "write_bytes": 24.0}}}
    (tmp_path / "profiles" / "w_traffic.json").write_text(json.dumps(rec))
    b.ROOT = str(tmp_path)
    assert b.profiled_traffic("k", "w") == 1024.0
    assert b.profiled_traffic("k", "other") is None
    assert b.profiled_traffic("other", "w") is None
    first = tmp_path / srcs[0]
    first.write_text(first.read_text() + "\n// edited\n")
    assert b.profiled_traffic("k", "w") is None
