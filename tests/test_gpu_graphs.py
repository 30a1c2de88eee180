"""The multi-launch entry points (low-rank branch, act-order layers, W4A8) under
HIP graph capture: one call captured, replayed several times with eager work and
synchronizations between the replays, every replay equal to the eager result bit
for bit."""
import numpy as np
import pytest

import workloads
from gpu_cases import say, to_dev

pytestmark = pytest.mark.gpu


def _replays_match(torch, call, out, replays=4):
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        call()
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    torch.cuda.synchronize()
    for i in range(replays):
        out.fill_(float("nan"))
        noise = torch.randn(1 << 20, device="cuda").sum()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(noise)
        assert torch.equal(out, eager), f"replay {i}"


@pytest.mark.parametrize("M", [1, 16, 200])
def test_lowrank_graph_replays(gpu_lib, M):
    import torch
    N, K, r = 300, 1024, 64
    W, x, _ = workloads.make(3, M=M, N=N, K=K)
    q = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=400)
    packed = gpu_lib.pack(q["codes"])
    L1, L2 = workloads.lowrank_factors(7, r, N, K)
    xd, L1d, L2d = to_dev(x, torch), to_dev(L1, torch), to_dev(L2, torch)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(gpu_lib.linear_lowrank_workspace_bytes(M, N, K, r), 1), dtype=torch.uint8, device="cuda")
    say(f"[graph lowrank] M={M}")
    _replays_match(torch, lambda: gpu_lib.linear_lowrank(xd, packed, q["scales"], q["zeros"], L1d, L2d, q["row_ptr"],
                                                         q["col"], q["val"], out=out, out_dtype=torch.float32,
                                                         workspace=ws), out)


@pytest.mark.parametrize("M", [1, 16, 200])
def test_lowrank_graph_replays_new_inputs(gpu_lib, M):
    """A low-rank product captured once: before each replay new activations are
    copied into the captured input, and every replay must equal an eager call on
    them bit for bit (a t left from the previous replay would differ)."""
    import torch
    N, K, r = 300, 1024, 64
    W, _, _ = workloads.make(3, M=M, N=N, K=K)
    q = gpu_lib.quantize_rtn(to_dev(W, torch), sparse_k=400)
    packed = gpu_lib.pack(q["codes"])
    L1, L2 = workloads.lowrank_factors(7, r, N, K)
    L1d, L2d = to_dev(L1, torch), to_dev(L2, torch)
    xd = torch.empty((M, K), dtype=torch.float16, device="cuda")
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(gpu_lib.linear_lowrank_workspace_bytes(M, N, K, r), 1), dtype=torch.uint8, device="cuda")

    def call(o, w):
        return gpu_lib.linear_lowrank(xd, packed, q["scales"], q["zeros"], L1d, L2d, q["row_ptr"], q["col"],
                                      q["val"], out=o, out_dtype=torch.float32, workspace=w)

    say(f"[graph lowrank new inputs] M={M}")
    stream = torch.cuda.Stream()
    xd.copy_(to_dev(workloads.random_x(50, M, K), torch))
    with torch.cuda.stream(stream):
        call(out, ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call(out, ws)
    torch.cuda.synchronize()
    ws2 = torch.empty_like(ws)
    for i in range(4):
        xd.copy_(to_dev(workloads.random_x(60 + i, M, K), torch))
        eager = call(torch.empty_like(out), ws2)
        torch.cuda.synchronize()
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"


@pytest.mark.parametrize("M", [1, 40, 200])
def test_act_order_graph_replays(gpu_lib, M):
    import torch
    N, K = 300, 1024
    W, x, _ = workloads.make(3, M=M, N=N, K=K)
    perm = to_dev(workloads.channel_permutation(8, K), torch)
    q = gpu_lib.quantize_rtn_act_order(to_dev(W, torch), perm, sparse_k=400)
    packed = gpu_lib.pack(q["codes"])
    xd = to_dev(x, torch)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.linear_act_order_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    say(f"[graph act-order] M={M}")
    _replays_match(torch, lambda: gpu_lib.linear_act_order(xd, perm, packed, q["scales"], q["zeros"], q["row_ptr"],
                                                           q["col"], q["val"], out=out, out_dtype=torch.float32,
                                                           workspace=ws), out)


@pytest.mark.parametrize("M", [1, 130])
def test_w4a8_graph_replays(gpu_lib, M):
    import torch
    N, K = 300, 1024
    W, x, _ = workloads.make(4, M=M, N=N, K=K)
    o = to_dev(workloads.x_outlier_channels(4, M=M, N=N, K=K), torch)
    q = gpu_lib.quantize_rtn(to_dev(W, torch))
    packed = gpu_lib.pack(q["codes"])
    xd = to_dev(x, torch)
    out = torch.empty((M, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.linear_w4a8_workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    say(f"[graph w4a8] M={M}")
    _replays_match(torch, lambda: gpu_lib.linear_w4a8(xd, o, packed, q["scales"], q["zeros"], out=out,
                                                      out_dtype=torch.float32, workspace=ws),
                   out)
