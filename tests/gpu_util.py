"""Helpers for the GPU parity tests: run the HIP library through its C ABI on
canary-filled buffers and compare with the CPU oracle byte for byte."""
from __future__ import annotations

import sys
from fractions import Fraction

import numpy as np
import pytest

import brute
import oracle

torch = pytest.importorskip("torch")
import lossless_bf16_tensor_exp_amd as ciera  # noqa: E402

GUARD = 256           # guard bytes on each side of every output buffer
CANARY = 0xA5
K0 = float.fromhex("0x1.a610ca4a234eep+9")


def say(*args):
    print(*args, file=sys.stderr, flush=True)


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    ciera.load_library()  # raises if the HIP library is not built


def _guarded_bytes(n, fill=CANARY):
    buf = torch.full((n + 2 * GUARD,), fill, dtype=torch.uint8, device="cuda")
    return buf, buf[GUARD:GUARD + n]


def _check_guards(host, n, what):
    assert (host[:GUARD] == CANARY).all(), f"{what}: write before the buffer"
    assert (host[GUARD + n:] == CANARY).all(), f"{what}: write after the buffer"


def oracle_encode(x, B=0, cache=None, e0=-1):
    """The oracle's 3-bit encode; from 2^24 values on, its chunk-parallel
    driver on the host's cores (the same bytes as the single-threaded
    encode, which the CPU tests pin)."""
    import os
    threads = min(16, os.cpu_count() or 1) if x.size >= (1 << 24) else 0
    return oracle.encode(x, B, cache, e0, threads=threads)


def window_tie(x, e0_a, e0_b):
    """Where the GPU (FP64 sums in its own order) and the oracle (exact) may
    pick different window bases: the exact variance lies within a relative
    2^-30 of the threshold K0 4^k between two adjacent bases, or it is
    cancellation-dominated (at most 2^-30 of the mean square about the GPU's
    shift K = x[0], or 0 if x[0] is not finite), where FP64 sums lose it."""
    var, nf = oracle.variance(x)
    if nf < 2:
        return False
    nf, s1, s2 = oracle.exact_moments(x)
    k_ = int(x[0]) if x.size and ((int(x[0]) >> 7) & 0xFF) != 255 else 0
    shift = brute.exact_value(k_)
    sdd = s2 - 2 * shift * s1 + nf * shift * shift  # sum of (v - K)^2
    if var * (nf - 1) <= sdd / 2 ** 30:
        return True
    if abs(e0_a - e0_b) != 1:
        return False
    t = Fraction(K0) * Fraction(4) ** (max(e0_a, e0_b) - 127)
    return abs(var - t) <= t / 2 ** 30


def exps(x):
    return ((x >> 7) & 0xFF).astype(np.uint8)


def gpu_encode(x, B=0, cache=None, e0=-1, stream=None, plan_groups=0):
    """Encode uint16 array x on the GPU.  Returns (stream bytes, cache after)."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.ciera_max_encoded_size(n, B) if B else ciera.zip3_max_encoded_size(n)
    ws_n = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    buf, out = _guarded_bytes(cap)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    cd = None
    if B:
        cbuf, cd = _guarded_bytes(n)
        cd.copy_(torch.from_numpy(cache))
        ciera.ciera_encode(xd, B, cd, out, ws, size, e0, stream, plan_groups)
    else:
        ciera.zip3_encode(xd, out, ws, size, e0, stream, plan_groups)
    torch.cuda.synchronize()
    assert ciera.ciera_read_error(ws) == 0
    sz = int(size.item())
    assert 0 < sz <= cap
    host = buf.cpu().numpy()
    _check_guards(host, cap, "stream")
    assert (host[GUARD + sz:GUARD + cap] == CANARY).all(), "write past the stream's end"
    new_cache = None
    if B:
        ch = cbuf.cpu().numpy()
        _check_guards(ch, n, "sender cache")
        new_cache = ch[GUARD:GUARD + n].copy()
    return host[GUARD:GUARD + sz].copy(), new_cache


def gpu_decode(stream_bytes, n, B=0, cache=None, in_size=None):
    """Decode on the GPU.  Returns (values uint16, cache after, device status)."""
    inp = torch.from_numpy(np.ascontiguousarray(stream_bytes)).cuda()
    in_size = stream_bytes.size if in_size is None else in_size
    ybuf, y = _guarded_bytes(2 * n)
    ws_n = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    yv = y.view(torch.int16)
    cd = None
    if B:
        cbuf, cd = _guarded_bytes(n)
        cd.copy_(torch.from_numpy(cache))
        ciera.ciera_decode(inp, in_size, yv, B, cd, ws)
    else:
        ciera.zip3_decode(inp, in_size, yv, ws)
    torch.cuda.synchronize()
    status = ciera.ciera_read_error(ws)
    host = ybuf.cpu().numpy()
    _check_guards(host, 2 * n, "y")
    new_cache = None
    if B:
        ch = cbuf.cpu().numpy()
        _check_guards(ch, n, "receiver cache")
        new_cache = ch[GUARD:GUARD + n].copy()
    return host[GUARD:GUARD + 2 * n].copy().view(np.uint16), new_cache, status


def _first_diff(a, b):
    m = min(a.size, b.size)
    d = np.flatnonzero(a[:m] != b[:m])
    return int(d[0]) if d.size else m


def check_encode(x, B=0, cache=None, e0=-1, stream=None, plan_groups=0):
    """GPU encode == oracle encode, byte for byte (and caches).  Where the
    window base differs, both choices must straddle a threshold within the
    FP64 summation error, and the rest must equal the oracle run at the GPU's
    window base.  Returns (stream, oracle stats)."""
    g_stream, g_cache = gpu_encode(x, B, cache, e0, stream, plan_groups)
    o_cache = cache.copy() if B else None
    o_stream, o_st = oracle_encode(x, B, o_cache, e0)
    if g_stream.tobytes() != o_stream.tobytes() and e0 < 0 and int(g_stream[7]) != o_st["E0"]:
        assert window_tie(x, int(g_stream[7]), o_st["E0"]), \
            f"window base differs away from a threshold: gpu {g_stream[7]} oracle {o_st['E0']}"
        o_cache = cache.copy() if B else None
        o_stream, o_st = oracle_encode(x, B, o_cache, int(g_stream[7]))
    if g_stream.tobytes() != o_stream.tobytes():
        i = _first_diff(g_stream, o_stream)
        raise AssertionError(f"stream differs from the oracle at byte {i} of {o_stream.size} "
                             f"(gpu size {g_stream.size}): gpu {g_stream[i:i + 16]} oracle {o_stream[i:i + 16]}")
    if B:
        assert np.array_equal(g_cache, o_cache), "sender cache differs from the oracle's"
        assert np.array_equal(g_cache, exps(x))
    return g_stream, o_st


def check_roundtrip(stream_bytes, x, B=0, cache=None):
    y, c, st = gpu_decode(stream_bytes, x.size, B, cache)
    assert st == 0, f"decode reported status {st}"
    if not np.array_equal(y, x):
        i = int(np.flatnonzero(y != x)[0])
        raise AssertionError(f"decode differs at value {i}: {y[i]:#06x} vs {x[i]:#06x}")
    if B:
        assert np.array_equal(c, exps(x)), "receiver cache is not the decoded exponents"
    return c


def gpu_encode_e0(x, e0_src, e0_offset=0, raw=False):
    """Single-read zip3 encode with the window base read from byte
    ``e0_offset`` of the uint8 device tensor ``e0_src``.  Returns (stream bytes
    or None, device status); with ``raw``, (whole output buffer, *out_size,
    device status) whatever the status."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.zip3_max_encoded_size(n)
    buf, out = _guarded_bytes(cap)
    ws = torch.empty(ciera.zip3_workspace_size(n), dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    ciera.zip3_encode_e0(xd, e0_src, out, ws, size, e0_offset)
    torch.cuda.synchronize()
    status = ciera.ciera_read_error(ws)
    host = buf.cpu().numpy()
    _check_guards(host, cap, "stream")
    if raw:
        return host[GUARD:GUARD + cap].copy(), int(size.item()), status
    if status:
        return None, status
    sz = int(size.item())
    assert 0 < sz <= cap
    assert (host[GUARD + sz:GUARD + cap] == CANARY).all(), "write past the stream's end"
    return host[GUARD:GUARD + sz].copy(), 0


def check_encode_e0(x, e0):
    """Single-read encode at window base e0 == oracle encode at e0, byte for byte."""
    src = torch.tensor([e0], dtype=torch.uint8, device="cuda")
    g, st = gpu_encode_e0(x, src)
    assert st == 0, f"single-read encode reported status {st}"
    o, _ = oracle_encode(x, 0, None, e0)
    if g.tobytes() != o.tobytes():
        i = _first_diff(g, o)
        raise AssertionError(f"single-read stream differs from the oracle at byte {i} of {o.size} "
                             f"(gpu size {g.size}): gpu {g[i:i + 16]} oracle {o[i:i + 16]}")
    return g


def gpu_encode_e0_ciera(x, B, cache, e0_src, e0_offset=0):
    """Single-read ciera encode: the window base from byte ``e0_offset`` of
    the uint8 device tensor ``e0_src``, the sender cache ``cache`` (n bytes,
    updated on the GPU).  Returns (stream bytes or None, device status,
    cache after)."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.ciera_max_encoded_size(n, B)
    buf, out = _guarded_bytes(cap)
    ws = torch.empty(ciera.ciera_workspace_size(n, B), dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    cbuf, cd = _guarded_bytes(n)
    cd.copy_(torch.from_numpy(cache))
    ciera.ciera_encode_e0(xd, B, cd, e0_src, out, ws, size, e0_offset)
    torch.cuda.synchronize()
    status = ciera.ciera_read_error(ws)
    host = buf.cpu().numpy()
    _check_guards(host, cap, "stream")
    ch = cbuf.cpu().numpy()
    _check_guards(ch, n, "sender cache")
    new_cache = ch[GUARD:GUARD + n].copy()
    if status:
        return None, status, new_cache
    sz = int(size.item())
    assert 0 < sz <= cap
    assert (host[GUARD + sz:GUARD + cap] == CANARY).all(), "write past the stream's end"
    return host[GUARD:GUARD + sz].copy(), 0, new_cache


def check_encode_e0_ciera(x, B, cache, e0):
    """Single-read ciera encode at window base e0 == oracle ciera encode at
    e0, stream and sender cache, byte for byte."""
    src = torch.tensor([e0], dtype=torch.uint8, device="cuda")
    g, st, gc = gpu_encode_e0_ciera(x, B, cache.copy(), src)
    assert st == 0, f"single-read ciera encode reported status {st}"
    oc = cache.copy()
    o, _ = oracle_encode(x, B, oc, e0)
    if g.tobytes() != o.tobytes():
        i = _first_diff(g, o)
        raise AssertionError(f"single-read ciera stream differs from the oracle at byte {i} of {o.size} "
                             f"(gpu size {g.size}): gpu {g[i:i + 16]} oracle {o[i:i + 16]}")
    assert np.array_equal(gc, oc), "sender cache differs from the oracle's"
    return g


def exps_as_bf16(e):
    """BF16 patterns whose exponent fields are the bytes e (sign and mantissa
    zero): a tensor whose block hashes stand for the exponent cache e."""
    return (np.asarray(e, dtype=np.uint16) << 7).astype(np.uint16)


def gpu_encode_hashed(x, B, hash_cache):
    """Hash-sender encode on the GPU.  Returns (stream bytes, hash cache after
    as a (blocks, 2) uint64 array)."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.ciera_max_encoded_size(n, B)
    buf, out = _guarded_bytes(cap)
    ws = torch.empty(ciera.ciera_workspace_size(n, B), dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    hb = ciera.ciera_hash_cache_size(n, B)
    hbuf, hd = _guarded_bytes(hb)
    hd.copy_(torch.from_numpy(np.ascontiguousarray(hash_cache).view(np.uint8).reshape(-1)))
    ciera.ciera_encode_hashed(xd, B, hd, out, ws, size)
    torch.cuda.synchronize()
    assert ciera.ciera_read_error(ws) == 0
    sz = int(size.item())
    assert 0 < sz <= cap
    host = buf.cpu().numpy()
    _check_guards(host, cap, "stream")
    assert (host[GUARD + sz:GUARD + cap] == CANARY).all(), "write past the stream's end"
    hh = hbuf.cpu().numpy()
    _check_guards(hh, hb, "hash cache")
    return host[GUARD:GUARD + sz].copy(), hh[GUARD:GUARD + hb].copy().view(np.uint64).reshape(-1, 2)


def check_encode_hashed(x, B, prev_exps):
    """Hash-sender encode against a hash cache holding the hashes of
    prev_exps == the oracle's exact-cache encode from prev_exps, byte for
    byte, and the cache afterwards holds x's block hashes."""
    hc = oracle.block_hashes(exps_as_bf16(prev_exps), B)
    g, hc_after = gpu_encode_hashed(x, B, hc)
    o_cache = np.ascontiguousarray(prev_exps, dtype=np.uint8).copy()
    o, st = oracle_encode(x, B, o_cache, -1)
    if g.tobytes() != o.tobytes() and int(g[7]) != st["E0"]:
        assert window_tie(x, int(g[7]), st["E0"]), f"window base: gpu {g[7]} oracle {st['E0']}"
        o_cache = np.ascontiguousarray(prev_exps, dtype=np.uint8).copy()
        o, st = oracle_encode(x, B, o_cache, int(g[7]))
    if g.tobytes() != o.tobytes():
        i = _first_diff(g, o)
        raise AssertionError(f"hash-sender stream differs from the oracle at byte {i} of {o.size} "
                             f"(gpu size {g.size}): gpu {g[i:i + 16]} oracle {o[i:i + 16]}")
    assert np.array_equal(hc_after, oracle.block_hashes(x, B)), "hash cache after encode"
    return g, st


def gpu_encode_rans(x, B=0, cache=None):
    """rANS-mode encode on the GPU.  Returns (stream bytes, cache after)."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.rans_max_encoded_size(n, B)
    buf, out = _guarded_bytes(cap)
    ws = torch.empty(ciera.rans_workspace_size(n, B), dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    cd = None
    if B:
        cbuf, cd = _guarded_bytes(n)
        cd.copy_(torch.from_numpy(cache))
        ciera.ciera_encode_rans(xd, B, cd, out, ws, size)
    else:
        ciera.zip3_encode_rans(xd, out, ws, size)
    torch.cuda.synchronize()
    assert ciera.ciera_read_error(ws) == 0
    sz = int(size.item())
    assert 0 < sz <= cap
    host = buf.cpu().numpy()
    _check_guards(host, cap, "stream")
    assert (host[GUARD + sz:GUARD + cap] == CANARY).all(), "write past the stream's end"
    new_cache = None
    if B:
        ch = cbuf.cpu().numpy()
        _check_guards(ch, n, "sender cache")
        new_cache = ch[GUARD:GUARD + n].copy()
    return host[GUARD:GUARD + sz].copy(), new_cache


def gpu_decode_rans(stream_bytes, n, B=0, cache=None, extra=0):
    """rANS-mode decode on the GPU, from a buffer holding the stream and
    ``extra`` more bytes (not part of it).  Returns (values, cache after,
    status)."""
    if extra:
        tail = np.random.default_rng(extra).integers(0, 256, extra, dtype=np.uint8)
        stream_bytes = np.concatenate([stream_bytes, tail])
    inp = torch.from_numpy(np.ascontiguousarray(stream_bytes)).cuda()
    ybuf, y = _guarded_bytes(2 * n)
    ws_n = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda")
    yv = y.view(torch.int16)
    cd = None
    if B:
        cbuf, cd = _guarded_bytes(n)
        cd.copy_(torch.from_numpy(cache))
        ciera.ciera_decode_rans(inp, stream_bytes.size, yv, B, cd, ws)
    else:
        ciera.zip3_decode_rans(inp, stream_bytes.size, yv, ws)
    torch.cuda.synchronize()
    status = ciera.ciera_read_error(ws)
    host = ybuf.cpu().numpy()
    _check_guards(host, 2 * n, "y")
    new_cache = None
    if B:
        ch = cbuf.cpu().numpy()
        _check_guards(ch, n, "receiver cache")
        new_cache = ch[GUARD:GUARD + n].copy()
    return host[GUARD:GUARD + 2 * n].copy().view(np.uint16), new_cache, status


def check_rans(x, B=0, cache=None):
    """GPU rANS encode == oracle rANS encode byte for byte (and the sender
    caches), and GPU decode returns x (and the receiver cache).  Returns the
    stream."""
    g, gc = gpu_encode_rans(x, B, cache)
    oc = cache.copy() if B else None
    o, _ = oracle.encode_rans(x, B, oc)
    if g.tobytes() != o.tobytes():
        i = _first_diff(g, o)
        raise AssertionError(f"rANS stream differs from the oracle at byte {i} of {o.size} "
                             f"(gpu size {g.size}): gpu {g[i:i + 16]} oracle {o[i:i + 16]}")
    if B:
        assert np.array_equal(gc, oc), "sender cache differs from the oracle's"
    y, rc, st = gpu_decode_rans(g, x.size, B, cache.copy() if B else None, extra=256)
    assert st == 0, f"rANS decode reported status {st}"
    if not np.array_equal(y, x):
        i = int(np.flatnonzero(y != x)[0])
        raise AssertionError(f"rANS decode differs at value {i}: {y[i]:#06x} vs {x[i]:#06x}")
    if B:
        assert np.array_equal(rc, exps(x)), "receiver cache is not the decoded exponents"
    return g
