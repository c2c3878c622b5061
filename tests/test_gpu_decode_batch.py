"""Batch decodes (zip3_decode_batch, ciera_decode_batch): k streams of one n
(and B) decoded in one launch, as a rank decodes the shards its peers sent.
Every stream comes from the oracle's encoder; each output must equal the
peer's tensor and each receiver cache its exponents, with guard bytes intact
around every output and cache, in_size given as the buffer's size (larger
than the stream), a workspace reused by a smaller batch, and one malformed
stream among well-formed ones."""
import numpy as np
import pytest

from gpu_util import GUARD, _check_guards, _guarded_bytes, exps, oracle_encode, require_gpu, say
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")
import lossless_bf16_tensor_exp_amd as ciera  # noqa: E402

pytestmark = pytest.mark.gpu

PAD = 384  # bytes of buffer after each stream: in_size is the buffer's size


def _peers(n, k, B, seed):
    """k peers' tensors of n values, the receiver caches (each peer's
    previous exponents, perturbed) and the oracle's streams."""
    rng = np.random.default_rng(seed)
    xs, caches, streams = [], [], []
    for _ in range(k):
        x = wl.mixed_small(rng, n)
        cache = wl.perturbed_cache(rng, x, 0.01) if B else None
        s, _ = oracle_encode(x, B, cache.copy() if B else None)
        xs.append(x)
        caches.append(cache)
        streams.append(s)
    return xs, caches, streams


def _batch(streams, n, B, caches, ws=None):
    """Decode the streams in one batch call into guarded buffers; returns
    (values, caches after, status)."""
    k = len(streams)
    inps, sizes = [], []
    for s in streams:
        buf = np.zeros(s.size + PAD, dtype=np.uint8)
        buf[:s.size] = s
        inps.append(torch.from_numpy(buf).cuda())
        sizes.append(buf.size)
    ybufs, ys, cbufs, cds = [], [], [], []
    for i in range(k):
        ybuf, y = _guarded_bytes(2 * n)
        ybufs.append(ybuf)
        ys.append(y.view(torch.int16))
        if B:
            cbuf, cd = _guarded_bytes(n)
            cd.copy_(torch.from_numpy(caches[i]))
            cbufs.append(cbuf)
            cds.append(cd)
    if ws is None:
        ws = torch.empty(ciera.decode_batch_workspace_size(n, k), dtype=torch.uint8, device="cuda")
    if B:
        ciera.ciera_decode_batch(inps, sizes, ys, B, cds, ws)
    else:
        ciera.zip3_decode_batch(inps, sizes, ys, ws)
    torch.cuda.synchronize()
    status = ciera.ciera_read_error(ws)
    vals, new_caches = [], []
    for i in range(k):
        host = ybufs[i].cpu().numpy()
        _check_guards(host, 2 * n, f"y[{i}]")
        vals.append(host[GUARD:GUARD + 2 * n].copy().view(np.uint16))
        if B:
            ch = cbufs[i].cpu().numpy()
            _check_guards(ch, n, f"receiver cache[{i}]")
            new_caches.append(ch[GUARD:GUARD + n].copy())
    return vals, new_caches, status


CASES = [  # (n, k, B)
    (0, 2, 0), (1000, 1, 0), (1000, 5, 0), (1 << 20, 3, 0), (33 * 65536 + 77, 3, 0), (65536 * 3 + 8, 16, 0),
    (0, 2, 256), (1000, 4, 64), (1 << 20, 3, 256), (1 << 20, 16, 512), (33 * 65536 + 77, 3, 64),
    (5 * 65536 + 1, 2, 32768), (40 * 65536, 2, 65536),
]


@pytest.mark.parametrize("n,k,B", CASES)
def test_batch_decode_equals_every_peer(n, k, B):
    require_gpu()
    say(f"decode batch n={n} k={k} B={B}")
    xs, caches, streams = _peers(n, k, B, seed=1000 * k + n % 997 + B)
    vals, new_caches, status = _batch(streams, n, B, caches)
    assert status == 0, status
    for i in range(k):
        assert np.array_equal(vals[i], xs[i]), f"stream {i}"
        if B:
            assert np.array_equal(new_caches[i], exps(xs[i])), f"receiver cache {i}"


def test_batch_workspace_reused_by_a_smaller_batch():
    require_gpu()
    n, B = 3 * 65536 + 1000, 128
    say(f"decode batch workspace reuse n={n}")
    ws = torch.empty(ciera.decode_batch_workspace_size(n, 6), dtype=torch.uint8, device="cuda")
    for k in (6, 2):
        xs, caches, streams = _peers(n, k, B, seed=77 + k)
        vals, new_caches, status = _batch(streams, n, B, caches, ws)
        assert status == 0, (k, status)
        for i in range(k):
            assert np.array_equal(vals[i], xs[i]) and np.array_equal(new_caches[i], exps(xs[i])), (k, i)


@pytest.mark.parametrize("B", [0, 256])
def test_one_malformed_stream_among_well_formed_ones(B):
    require_gpu()
    n, k, bad = (1 << 20) + 4096, 4, 2
    say(f"decode batch with stream {bad} malformed, B={B}")
    xs, caches, streams = _peers(n, k, B, seed=5 + B)
    streams[bad] = streams[bad].copy()
    streams[bad][0] ^= 0xFF  # magic
    vals, new_caches, status = _batch(streams, n, B, caches)
    assert status == ciera.STATUS_CODES["CIERA_ERR_FORMAT"], status
    for i in range(k):
        if i == bad:
            continue
        assert np.array_equal(vals[i], xs[i]), f"stream {i}"
        if B:
            assert np.array_equal(new_caches[i], exps(xs[i])), f"receiver cache {i}"
