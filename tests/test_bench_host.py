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


def test_trace_durations_pairs_labels_with_bench_dispatches(tmp_path):
    """The kernel-trace parser keeps only the library's and calibration
    kernels (namespace bq), in dispatch order, pairs them one to one with the
    trace child's labels, and refuses a count mismatch."""
    b = _bench()
    rows = [  # (dispatch id, name, start ns, end ns), out of order on purpose
        (3, "void bq::(anonymous namespace)::gemv_kernel<4, 1, 1, 4, 2, true>(...)", 5000, 9500),
        (1, "void bq::(anonymous namespace)::quantize_rows_vec<2>(...)", 1000, 31000),
        (2, "void at::native::vectorized_elementwise_kernel<...>", 31000, 31500),
        (4, "void bq::calib::read_stream_kernel(uint4 const*, long, unsigned int*)", 10000, 14000),
        (5, "void bq::(anonymous namespace)::gemv_kernel<4, 1, 1, 4, 2, true>(...)", 20000, 24500),
    ]
    p = tmp_path / "bench_kernel_trace.csv"
    with open(p, "w") as fh:
        fh.write('"Kind","Dispatch_Id","Kernel_Name","Start_Timestamp","End_Timestamp"\n')
        for d, n, s, e in rows:
            fh.write(f'"KERNEL_DISPATCH",{d},"{n}",{s},{e}\n')
    got = b.trace_durations(str(p), ["quantize_rows", "gemm_w4a8_m1", "read", "gemm_w4a8_m1"])
    assert got == {"quantize_rows": [30.0], "gemm_w4a8_m1": [4.5, 4.5], "read": [4.0]}
    import pytest

    with pytest.raises(ValueError):
        b.trace_durations(str(p), ["quantize_rows", "gemm_w4a8_m1"])
    st = b.stats([1.0, 2.0, 3.0, 4.0, 100.0])
    assert st["us"] == 3.0 and st["n"] == 5 and st["us_min"] == 1.0
