"""The codec inside a captured HIP graph (torch.cuda.CUDAGraph): encode and
decode launch only kernels (no memsets, no host synchronisation; every reset
of workspace words is done by a kernel), so a graph of one step can be
replayed.  Each replay is checked against the eager result, with eager work
and synchronisations between the replays."""
import numpy as np
import pytest

from gpu_util import ciera, require_gpu, say, torch
from lossless_bf16_tensor_exp_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _bufs(n, B):
    cap = ciera.ciera_max_encoded_size(n, B) if B else ciera.zip3_max_encoded_size(n)
    wsz = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    return (torch.zeros(cap, dtype=torch.uint8, device="cuda"), torch.zeros(wsz, dtype=torch.uint8, device="cuda"),
            torch.zeros(wsz, dtype=torch.uint8, device="cuda"), torch.zeros(1, dtype=torch.int64, device="cuda"))


@pytest.mark.parametrize("B", [0, 256])
def test_graph_replays_match_eager(B):
    d = wl.workload1()
    x0, x1 = d["iters"]
    n = x0.size
    say(f"graph B={B} n={n}")
    xs = [torch.from_numpy(a.view(np.int16)).cuda() for a in (x0, x1)]
    e0 = torch.from_numpy(((x0 >> 7) & 0xFF).astype(np.uint8)).cuda()
    # eager reference: encode x1 against E(x0), decode it
    out, ws_e, ws_d, size = _bufs(n, B)
    y = torch.empty(n, dtype=torch.int16, device="cuda")
    send, recv = e0.clone(), e0.clone()
    if B:
        ciera.ciera_encode(xs[1], B, send, out, ws_e, size)
    else:
        ciera.zip3_encode(xs[1], out, ws_e, size)
    torch.cuda.synchronize()
    sz = int(size.item())
    ref = out[:sz].clone()
    if B:
        ciera.ciera_decode(out, sz, y, B, recv, ws_d)
    else:
        ciera.zip3_decode(out, sz, y, ws_d)
    torch.cuda.synchronize()
    assert torch.equal(y, xs[1])

    # capture one step on a side stream
    out2, ws_e2, ws_d2, size2 = _bufs(n, B)
    y2 = torch.empty_like(y)
    send2, recv2 = e0.clone(), e0.clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            s = torch.cuda.current_stream()
            if B:
                ciera.ciera_encode(xs[1], B, send2, out2, ws_e2, size2, stream=s)
                ciera.ciera_decode(out2, sz, y2, B, recv2, ws_d2, stream=s)
            else:
                ciera.zip3_encode(xs[1], out2, ws_e2, size2, stream=s)
                ciera.zip3_decode(out2, sz, y2, ws_d2, stream=s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(5):
        # eager work between replays: reset caches and outputs, disturb memory
        send2.copy_(e0)
        recv2.copy_(e0)
        out2.fill_(0xA5)
        y2.fill_(-1)
        size2.fill_(-1)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(size2.item()) == sz, f"replay {r}: size"
        assert torch.equal(out2[:sz], ref), f"replay {r}: stream differs from the eager one"
        assert torch.equal(y2, xs[1]), f"replay {r}: decoded values"
        assert ciera.ciera_read_error(ws_e2) == 0 and ciera.ciera_read_error(ws_d2) == 0
        if B:
            assert np.array_equal(send2.cpu().numpy(), ((x1 >> 7) & 0xFF).astype(np.uint8)), f"replay {r}: cache"
        del junk
