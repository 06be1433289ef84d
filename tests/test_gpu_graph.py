"""The LM-head step captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed: the library's entry points allocate nothing, synchronise nothing
and enqueue no memset, so a captured step must replay the eager result
bitwise.  Each replay runs with its outputs cleared first and with eager
work and synchronisations between replays; every replay is compared with
the eager step.

Shapes: a ragged one (unsplit dgrad, edge tiles), the 128-token step (few
token logits kernel, split dgrad, two-per-CU wgrad) and the 1024-token step
(ping-pong logits kernel, split dgrad)."""
import pytest
import torch

import lm_head_fp32_amd as lmh

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lmh.lib()


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


@pytest.mark.parametrize("M,K,V", [(100, 520, 1000), (128, 4096, 32768), (1024, 8192, 32768)])
def test_step_graph_replays_match_eager(M, K, V):
    print(f"graph step M={M} K={K} V={V}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(1000 + M)
    x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    W = (0.02 * torch.randn(V, K, device="cuda", generator=g)).to(torch.bfloat16)
    tgt = torch.randint(0, V, (M,), device="cuda", dtype=torch.int32, generator=g)
    tgt[::20] = -100
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    loss = torch.empty((M,), dtype=torch.float32, device="cuda")
    stats = torch.empty((M, 4), dtype=torch.float32, device="cuda")
    mean = torch.empty((1,), dtype=torch.float32, device="cuda")
    inv = torch.empty((1,), dtype=torch.float32, device="cuda")
    dlog = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((V, K), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(lmh.lmhead_dgrad_workspace_bytes(M, K, V), 16), dtype=torch.uint8,
                     device="cuda")
    outs = (logits, loss, stats, mean, inv, dlog, dX, dW)

    def step():
        lmh.lmhead_logits(x, W, out=logits, out_dtype="fp32")
        lmh.lmhead_xent_fwd(logits, tgt, -100, loss=loss, stats=stats)
        lmh.lmhead_xent_mean(loss, tgt, -100, mean=mean, inv_nvalid=inv)
        lmh.lmhead_xent_bwd(logits, stats, tgt, inv, -100, dlogits=dlog, grad_dtype="bf16")
        lmh.lmhead_dgrad(dlog, W, dX=dX, dx_dtype="bf16", workspace=ws)
        lmh.lmhead_wgrad(dlog, x, dW=dW)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert torch.isfinite(mean).all().item()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(("logits", "loss", "stats", "mean", "inv", "dlogits", "dX",
                                    "dW"), outs, ref):
            assert torch.equal(_bits(got), _bits(want)), (rep, name)
        step()  # eager work between replays
        torch.cuda.synchronize()
    del graph


@pytest.mark.parametrize("M,K,V", [(100, 520, 1000), (128, 4096, 32768), (1024, 8192, 32768)])
def test_single_read_path_graph_replays_match_eager(M, K, V):
    """The single-read forms captured the same way: logits with the CE
    records from the GEMM epilogue, their merge, the mean, and the fused CE
    forward + backward (BF16 grads)."""
    print(f"graph single-read M={M} K={K} V={V}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(2000 + M)
    x = torch.randn(M, K, device="cuda", generator=g).to(torch.bfloat16)
    W = (0.02 * torch.randn(V, K, device="cuda", generator=g)).to(torch.bfloat16)
    tgt = torch.randint(0, V, (M,), device="cuda", dtype=torch.int32, generator=g)
    tgt[1::25] = -100
    logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
    part = torch.empty(((V + 255) // 256, M, 4), dtype=torch.float32, device="cuda")
    loss = torch.empty((M,), dtype=torch.float32, device="cuda")
    stats = torch.empty((M, 4), dtype=torch.float32, device="cuda")
    mean = torch.empty((1,), dtype=torch.float32, device="cuda")
    inv = torch.empty((1,), dtype=torch.float32, device="cuda")
    loss2 = torch.empty((M,), dtype=torch.float32, device="cuda")
    stats2 = torch.empty((M, 4), dtype=torch.float32, device="cuda")
    dlog = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")
    outs = (logits, part, loss, stats, mean, inv, loss2, stats2, dlog)

    def step():
        lmh.lmhead_logits_xent(x, W, tgt, -100, out=logits, part=part)
        lmh.lmhead_xent_merge(part, tgt, V, -100, loss=loss, stats=stats)
        lmh.lmhead_xent_mean(loss, tgt, -100, mean=mean, inv_nvalid=inv)
        lmh.lmhead_xent_fused(logits, tgt, inv, -100, dlogits=dlog, grad_dtype="bf16",
                              loss=loss2, stats=stats2)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    assert torch.isfinite(mean).all().item()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    names = ("logits", "part", "loss", "stats", "mean", "inv", "fused loss", "fused stats",
             "dlogits")
    for rep in range(3):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, want in zip(names, outs, ref):
            assert torch.equal(_bits(got), _bits(want)), (rep, name)
        step()
        torch.cuda.synchronize()
    del graph
