"""The one-shot calls of the Python binding (allocate, encode or decode,
return the stream and its size): streams equal the oracle's byte for byte,
decodes return the input, caches follow (ZipCCL digest, section 3.1: the
3-bit code; CIERA page, section 3.1: exponent reuse)."""
import numpy as np
import pytest

from gpu_util import exps, oracle_encode, require_gpu, say, window_tie
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def _same_as_oracle(g, x, B, cache_before):
    o_cache = cache_before.copy() if B else None
    o, st = oracle_encode(x, B, o_cache)
    if g.tobytes() != o.tobytes() and int(g[7]) != st["E0"]:
        assert window_tie(x, int(g[7]), st["E0"])
        o_cache = cache_before.copy() if B else None
        o, st = oracle_encode(x, B, o_cache, int(g[7]))
    assert g.tobytes() == o.tobytes(), "stream differs from the oracle's"
    return o_cache


def test_zip3_one_shot():
    from lossless_bf16_tensor_exp_amd.codec import zip3_decode_tensor, zip3_encode_tensor
    x = wl.workload1()["iters"][1][: 200_003]
    say(f"zip3 one-shot n={x.size}")
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    s, k = zip3_encode_tensor(xd)
    assert s.numel() == k
    _same_as_oracle(s.cpu().numpy(), x, 0, None)
    y = zip3_decode_tensor(s, x.size)
    assert torch.equal(y, xd)


def test_ciera_one_shot_two_iterations():
    from lossless_bf16_tensor_exp_amd.codec import ciera_decode_tensor, ciera_encode_tensor
    d = wl.workload1()
    x0, x1 = d["iters"]
    B = d["B"][0]
    say(f"ciera one-shot n={x0.size} B={B}")
    send = torch.zeros(x0.size, dtype=torch.uint8, device="cuda")
    recv = torch.zeros_like(send)
    host_cache = np.zeros(x0.size, dtype=np.uint8)
    for x in (x0, x1):
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        s, k = ciera_encode_tensor(xd, B, send)
        assert s.numel() == k
        host_cache = _same_as_oracle(s.cpu().numpy(), x, B, host_cache)
        assert np.array_equal(send.cpu().numpy(), exps(x))
        y = ciera_decode_tensor(s, x.size, B, recv)
        assert torch.equal(y, xd)
        assert torch.equal(recv, send)


def test_decode_of_a_damaged_stream_raises():
    from lossless_bf16_tensor_exp_amd import CieraError
    from lossless_bf16_tensor_exp_amd.codec import zip3_decode_tensor, zip3_encode_tensor
    x = wl.workload1()["iters"][0][: 70_000]
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    s, _ = zip3_encode_tensor(xd)
    bad = s.clone()
    bad[0] ^= 0xFF  # magic
    with pytest.raises(CieraError):
        zip3_decode_tensor(bad, x.size)
