"""The path captured in a HIP graph (torch.cuda.graph on the stream that ran
the warm-up) and replayed: quantize -> pack -> GEMMs on every kernel path,
with eager work and synchronizations between replays.  Every replay must give
the eager results bit for bit (the kernels are deterministic), which also
shows that no call of the path allocates, synchronizes or memsets inside the
capture.  One call splits K over workgroups (bq_gemm_splitk, 16 tiles,
K = 1024) with a workspace allocated and zeroed before the capture; the
graph replays the split kernel on it, and its per-tile counters must reset
themselves on every replay."""
import numpy as np
import pytest

from bit_mixed_precision_amd import synth
from gpu_util import banner, need_gpu, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return need_gpu()


def test_graph_replays_match_eager(dev):
    from bit_mixed_precision_amd import bq
    import torch

    banner("graph capture of quantize -> pack -> gemm")
    g = np.random.default_rng(90)
    W = to_dev(synth.fp16_normal(g, (512, 1024), 0.02), dev)
    X = to_dev(synth.fp16_normal(g, (96, 1024), 1.0), dev)
    A1 = to_dev(synth.int8_uniform(g, (1, 1024)), dev)

    def path(o):
        q4, s4 = bq.quantize_rows_bits(W, 4, o["q4"], o["s4"])
        bq.pack_int4(q4, o["p4"])
        qx, sx = bq.quantize_rows(X, o["qx"], o["sx"])
        bq.gemm(qx, o["p4"], 4, s4, out=o["c_tiled"], path="tiled")
        bq.gemm_splitk(qx, o["p4"], 4, s4, o["ws"], out=o["c_split"])
        bq.gemm_dual_scale(qx[:20], o["p4"], 4, s4, sx[:20], out=o["c_stream"], path="stream")
        bq.gemm(A1, o["p4"], 4, s4, out=o["c_gemv"], path="gemv")
        bq.gemm_act(qx, o["p4"], 4, s4, sx, act="gelu", out=o["c_act"])

    def buffers():
        return {
            "q4": torch.empty((512, 1024), dtype=torch.int8, device=dev),
            "s4": torch.empty((512,), dtype=torch.float16, device=dev),
            "p4": torch.empty((512, 512), dtype=torch.uint8, device=dev),
            "qx": torch.empty((96, 1024), dtype=torch.int8, device=dev),
            "sx": torch.empty((96,), dtype=torch.float16, device=dev),
            "c_tiled": torch.empty((96, 512), dtype=torch.float16, device=dev),
            "c_split": torch.empty((96, 512), dtype=torch.float16, device=dev),
            "ws": torch.zeros(bq.gemm_splitk_workspace_bytes(96, 512, 1024, 4), dtype=torch.uint8, device=dev),
            "c_stream": torch.empty((20, 512), dtype=torch.float16, device=dev),
            "c_gemv": torch.empty((1, 512), dtype=torch.float16, device=dev),
            "c_act": torch.empty((96, 512), dtype=torch.float16, device=dev),
        }

    eager = buffers()
    path(eager)
    torch.cuda.synchronize()
    ref = {k: v.cpu().clone() for k, v in eager.items()}

    gbuf = buffers()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        path(gbuf)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        path(gbuf)
    assert bq.gemm_splitk_workspace_bytes(96, 512, 1024, 4) > 0  # the call does split
    for rep in range(4):
        for k, v in gbuf.items():  # poison the outputs between replays
            if k != "ws":
                v.zero_()
        _ = (W.float() * 2).sum()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, v in gbuf.items():
            if k != "ws":
                assert torch.equal(v.cpu(), ref[k]), f"replay {rep}: {k} differs from eager"
        assert int(gbuf["ws"][:4096].count_nonzero()) == 0, "split-K counters not reset"
    assert torch.equal(gbuf["c_split"], gbuf["c_tiled"])
