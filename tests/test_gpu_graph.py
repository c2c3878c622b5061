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


@pytest.mark.parametrize("B", [0, 256])
def test_graph_replays_of_the_speculative_encode_and_the_batch_decode(B):
    """A captured speculative encode (40 chunks, hint in device memory) and a
    batch decode of two copies of its stream: replays with the hint set right
    and wrong between them (eager work) equal the eager regular encode, and
    both decodes give the input back."""
    rng = np.random.default_rng(3 + B)
    n = 40 * 65536 + 321
    x0 = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    x1 = x0.copy()
    wl.flip(x1, rng.choice(n, size=n // 300, replace=False))
    say(f"graph speculative encode + batch decode B={B} n={n}")
    xd = torch.from_numpy(x1.view(np.int16)).cuda()
    e0 = torch.from_numpy(((x0 >> 7) & 0xFF).astype(np.uint8)).cuda()
    out, ws_e, _, size = _bufs(n, B)
    send = e0.clone()
    if B:
        ciera.ciera_encode(xd, B, send, out, ws_e, size)
    else:
        ciera.zip3_encode(xd, out, ws_e, size)
    torch.cuda.synchronize()
    sz = int(size.item())
    ref = out[:sz].clone()
    right = int(ref[7].item())
    hint = torch.tensor([right], dtype=torch.uint8, device="cuda")

    out2, ws_e2, _, size2 = _bufs(n, B)
    ws_b = torch.zeros(ciera.decode_batch_workspace_size(n, 2), dtype=torch.uint8, device="cuda")
    ys = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(2)]
    send2 = e0.clone()
    recvs = [e0.clone() for _ in range(2)]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            s = torch.cuda.current_stream()
            if B:
                ciera.ciera_encode_spec(xd, B, send2, hint, out2, ws_e2, size2, stream=s)
                ciera.ciera_decode_batch([out2, out2], [sz, sz], ys, B, recvs, ws_b, stream=s)
            else:
                ciera.zip3_encode_spec(xd, hint, out2, ws_e2, size2, stream=s)
                ciera.zip3_decode_batch([out2, out2], [sz, sz], ys, ws_b, stream=s)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r, h in enumerate([right, right + 1, right, 255, right - 1, right]):
        send2.copy_(e0)
        for c in recvs:
            c.copy_(e0)
        out2.fill_(0xA5)
        for y in ys:
            y.fill_(-1)
        size2.fill_(-1)
        hint.fill_(h)
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert ciera.ciera_read_error(ws_e2) == 0 and ciera.ciera_read_error(ws_b) == 0, f"replay {r}"
        assert int(size2.item()) == sz, f"replay {r} (hint {h}): size"
        assert torch.equal(out2[:sz], ref), f"replay {r} (hint {h}): stream differs from the eager one"
        for y in ys:
            assert torch.equal(y, xd), f"replay {r}: decoded values"
        if B:
            want = ((x1 >> 7) & 0xFF).astype(np.uint8)
            assert np.array_equal(send2.cpu().numpy(), want), f"replay {r}: sender cache"
            for c in recvs:
                assert np.array_equal(c.cpu().numpy(), want), f"replay {r}: receiver cache"
        del junk
