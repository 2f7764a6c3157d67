"""Host logic of bench.py, on the CPU: the refusal to run on more than one GPU,
the buffer ring that spans more than twice the MALL, and the rule that the
committed HBM-traffic summary counts only for the kernel sources it was
taken from (comments and blank space aside)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_host_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_ring_spans_twice_the_mall():
    b = _bench()
    for nbytes in (1, 4096, 8 << 20, 100 << 20, 512 << 20, 600 << 20):
        n = b.ring_len(nbytes)
        assert n >= 2
        assert n * nbytes > 2 * b.MALL_BYTES
        # and not more than one buffer beyond what that needs
        assert n == 2 or (n - 2) * nbytes <= 2 * b.MALL_BYTES


def test_source_hash_ignores_comments_and_blank_space():
    b = _bench()
    assert b._code_only("int a = 1; // note\n") == b._code_only("int  a=1;/* other\n note */")
    assert b._code_only('f("a // b");') == b._code_only('f( "a // b" ) ;')
    assert b._code_only("a + 1;") != b._code_only("a - 1;")


def test_traffic_summary_follows_the_source_hash(monkeypatch):
    b = _bench()
    recorded = None
    for line in open(b.TRAFFIC_FILE):
        if line.startswith("source_sha256_16:"):
            recorded = line.split(":", 1)[1].strip()
    assert recorded is not None
    if recorded == b.tiled_source_hash():
        got = b.measured_traffic()
        assert isinstance(got, int)
        # at least the algorithmic bytes of the M = N = K = 4096 W4A8 launch
        assert got >= 4096 * 4096 + 4096 * 2048 + 2 * 4096 + 2 * 4096 * 4096
    # a source change (a different hash) voids the summary
    monkeypatch.setattr(b, "tiled_source_hash", lambda: "0" * 16)
    assert b.measured_traffic() is None
