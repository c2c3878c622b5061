"""The encode that allocates nothing (ciera_encode_noalloc, for callers that
cannot allocate device memory) against ciera_encode with a caller's
workspace: the same stream bytes, *out_size and sender cache, on calls in a
row that reuse the library's one scratch array (a larger input, then a
smaller one, then the largest allowed), and sizes above the limit refused
before anything is enqueued."""
import numpy as np
import pytest

from gpu_util import require_gpu, say
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")
import lossless_bf16_tensor_exp_amd as ciera  # noqa: E402

pytestmark = pytest.mark.gpu


def _pair(n, B, seed):
    """(x, the previous iteration's exponents) with some blocks changed."""
    rng = np.random.default_rng(seed)
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    prev = ((x >> 7) & 0xFF).astype(np.uint8)
    prev[rng.random(n) < 0.003] ^= 1
    return x, prev


def _both(x, prev, B):
    """Encode x against prev with both entry points; returns their (stream,
    size, cache) triples."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.ciera_max_encoded_size(n, B)
    res = []
    for noalloc in (True, False):
        out = torch.full((cap,), 0xA5, dtype=torch.uint8, device="cuda")
        size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
        cache = torch.from_numpy(prev).cuda()
        if noalloc:
            ciera.ciera_encode_noalloc(xd, B, cache, out, size)
            torch.cuda.synchronize()
        else:
            ws = torch.empty(ciera.ciera_workspace_size(n, B), dtype=torch.uint8, device="cuda")
            ciera.ciera_encode(xd, B, cache, out, ws, size)
            torch.cuda.synchronize()
            assert ciera.ciera_read_error(ws) == 0
        sz = int(size.item())
        assert 0 < sz <= cap
        res.append((out.cpu().numpy(), sz, cache.cpu().numpy()))
    return res


def test_noalloc_encode_equals_the_workspace_encode_on_calls_in_a_row():
    require_gpu()
    cases = [(40 * 65536 + 12345, 256, 1), (65536 + 77, 64, 2), (1000, 4096, 3),
             (ciera.NOALLOC_MAX_N, 512, 4)]
    for n, B, seed in cases:
        say(f"noalloc encode n={n} B={B}")
        x, prev = _pair(n, B, seed)
        (a, sa, ca), (b, sb, cb) = _both(x, prev, B)
        assert sa == sb, (n, B)
        assert a.tobytes() == b.tobytes(), (n, B)  # the stream and the bytes past it
        assert np.array_equal(ca, cb) and np.array_equal(ca, (x >> 7) & 0xFF)


def test_noalloc_encode_refuses_sizes_above_its_limit():
    require_gpu()
    n = ciera.NOALLOC_MAX_N + 1
    x = torch.zeros(8, dtype=torch.int16, device="cuda")  # never read: refused first
    out = torch.zeros(16, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    lib = ciera.load_library()
    import ctypes
    st = lib.ciera_encode_noalloc(ctypes.c_void_p(x.data_ptr()), n, 256, ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(out.data_ptr()), 1 << 62, ctypes.c_void_p(size.data_ptr()),
                                  None)
    assert st == ciera.STATUS_CODES["CIERA_ERR_WORKSPACE"]
    assert int(size.item()) == 0
