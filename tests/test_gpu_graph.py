"""The library's calls under HIP graph capture.

Every entry point only launches kernels on the stream it is given (no
allocation, no synchronisation, no memset), so a sequence of calls can be
captured once and replayed.  This captures MX QDQ with a rotation, quantize,
dequantize, NVFP4 QDQ and the GEMM into one graph (outputs allocated
beforehand), replays it three times with eager work and synchronisations
in between, and compares every replay bit for bit with the same calls run
eagerly.
"""
import numpy as np
import pytest

from _parity import to_gpu_bf16
from microscaling_quantize_dequantize_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mx():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from microscaling_quantize_dequantize_amd import binding
    return binding


def test_captured_calls_replay_like_eager(mx):
    import torch
    M, K = 256, 4096
    x = to_gpu_bf16(W.random_bf16((M, K), seed=11))
    R = to_gpu_bf16(W.hadamard_rotation(128))
    g = torch.tensor([448.0 * 6.0 / float(x.float().abs().max())], dtype=torch.float32, device="cuda")
    outs = {
        "qdq": torch.empty_like(x),
        "codes": torch.empty((M, K // 2), dtype=torch.uint8, device="cuda"),
        "scales": torch.empty((M, K // 32), dtype=torch.uint8, device="cuda"),
        "deq": torch.empty_like(x),
        "nv": torch.empty_like(x),
        "c": torch.empty((M, M), dtype=torch.bfloat16, device="cuda"),
    }

    def run():
        mx.mx_qdq(0, x, rot=R, dst=outs["qdq"])
        mx.mx_quantize(0, x, rot=R, codes=outs["codes"], scales=outs["scales"])
        mx.mx_dequantize(0, outs["codes"], outs["scales"], K, dst=outs["deq"])
        mx.mx_nvfp4_qdq(x, g, dst=outs["nv"])
        mx.mx_matmul(0, outs["codes"], outs["scales"], outs["codes"], outs["scales"], K, c=outs["c"])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = {k: v.clone() for k, v in outs.items()}

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()
    for rep in range(3):
        for v in outs.values():
            v.zero_()  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k in outs:
            assert torch.equal(outs[k].view(torch.uint8), eager[k].view(torch.uint8)), (rep, k)
