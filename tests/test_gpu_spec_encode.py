"""Speculative encodes (zip3_encode_spec, ciera_encode_spec) against the
oracle.  For hint bytes that are right, one binade off either way, 0, 249 and
out of range, the stream, *out_size and the sender cache must equal the
oracle's encode of the same input, whose window comes from the variance (and
so the regular GPU encode's); also with the hint read from the output buffer
itself (byte 7 of the previous iteration's stream) over three iterations, on
tensors small enough to take the regular encode, on inputs with non-finite
values (the variance sums' second pass), and when the waits between
workgroups are forced to give up."""
import numpy as np
import pytest

import oracle
from gpu_util import (GUARD, _check_guards, _guarded_bytes, check_encode, check_roundtrip, exps, oracle_encode,
                      require_gpu, say)
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")
import lossless_bf16_tensor_exp_amd as ciera  # noqa: E402

pytestmark = pytest.mark.gpu


def spec_encode(x, B, cache, hint=None, hint_src=None, hint_offset=0):
    """Speculative encode on the GPU into a guarded buffer.  Returns (stream,
    cache after, status)."""
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    cap = ciera.ciera_max_encoded_size(n, B) if B else ciera.zip3_max_encoded_size(n)
    wsz = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    obuf, out = _guarded_bytes(cap)
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    if hint_src is None:
        hint_src = torch.tensor([hint], dtype=torch.uint8, device="cuda")
    cd = None
    if B:
        cbuf, cd = _guarded_bytes(n)
        cd.copy_(torch.from_numpy(cache))
        ciera.ciera_encode_spec(xd, B, cd, hint_src, out, ws, size, hint_offset)
    else:
        ciera.zip3_encode_spec(xd, hint_src, out, ws, size, hint_offset)
    torch.cuda.synchronize()
    status = ciera.ciera_read_error(ws)
    host = obuf.cpu().numpy()
    _check_guards(host, cap, "stream buffer")
    sz = int(size.item())
    new_cache = None
    if B:
        ch = cbuf.cpu().numpy()
        _check_guards(ch, n, "sender cache")
        new_cache = ch[GUARD:GUARD + n].copy()
    return host[GUARD:GUARD + max(sz, 0)].copy(), new_cache, status


def _check(x, B, cache, hint):
    want, st = check_encode(x, B, cache.copy() if B else None)  # the regular GPU encode == the oracle
    got, new_cache, status = spec_encode(x, B, cache.copy() if B else None, hint)
    assert status == 0, status
    assert got.tobytes() == want.tobytes(), f"speculative stream differs (hint {hint}, E0 {int(want[7])})"
    if B:
        assert np.array_equal(new_cache, exps(x)), "sender cache"
    return want, st


HINTS = ["right", "low", "high", 0, 249, 250, 255]
BLOCKS = [0, 64, 256, 512, 4096, 32768, 65536]


@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("hint", HINTS)
def test_spec_encode_equals_the_oracle_for_every_hint(B, hint):
    require_gpu()
    seed = 100 * BLOCKS.index(B) + HINTS.index(hint)
    rng = np.random.default_rng(seed)
    n = (17 * 65536 + 1234) if seed % 2 else 40 * 65536
    # Gaussian at a random scale most of the time; the mixes with specials
    # (non-finite values) every third case
    x = wl.mixed_small(rng, n) if seed % 3 == 0 else wl.f32_to_bf16(
        rng.standard_normal(n, dtype=np.float32) * np.float32(10.0 ** rng.uniform(-4, 1)))
    cache = wl.perturbed_cache(rng, x, 0.01) if B else None
    right = oracle.choose_e0(x)
    h = {"right": right, "low": max(0, right - 1), "high": min(249, right + 1)}.get(hint, hint)
    say(f"spec encode n={n} B={B} hint={hint}->{h} E0={right}")
    _check(x, B, cache, h)


@pytest.mark.parametrize("B", [0, 256])
def test_spec_encode_hint_from_the_previous_stream(B):
    """Three iterations into one output buffer, each hinted by byte 7 of the
    stream the previous one left there; each equals the oracle's encode and
    decodes back."""
    require_gpu()
    rng = np.random.default_rng(7 + B)
    n = 33 * 65536 + 99
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    cap = ciera.ciera_max_encoded_size(n, B) if B else ciera.zip3_max_encoded_size(n)
    wsz = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    ws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    send = torch.zeros(n, dtype=torch.uint8, device="cuda")
    ocache = np.zeros(n, dtype=np.uint8)
    for it in range(3):
        if it:
            wl.flip(x, rng.choice(n, size=n // 500, replace=False))
        xd = torch.from_numpy(x.view(np.int16)).cuda()
        say(f"spec encode chain B={B} iteration {it}")
        if it == 0:  # no previous stream yet: the regular encode
            if B:
                ciera.ciera_encode(xd, B, send, out, ws, size)
            else:
                ciera.zip3_encode(xd, out, ws, size)
        elif B:
            ciera.ciera_encode_spec(xd, B, send, out, out, ws, size, 7)
        else:
            ciera.zip3_encode_spec(xd, out, out, ws, size, 7)
        torch.cuda.synchronize()
        assert ciera.ciera_read_error(ws) == 0
        sz = int(size.item())
        recv = ocache.copy()  # a receiver's cache before this iteration
        want, _ = oracle_encode(x, B, ocache if B else None)
        got = out[:sz].cpu().numpy()
        assert got.tobytes() == want.tobytes(), f"iteration {it}"
        if B:
            assert np.array_equal(send.cpu().numpy(), ocache)
    check_roundtrip(got, x, B, recv if B else None)


@pytest.mark.parametrize("B", [0, 512])
def test_spec_encode_of_a_small_tensor_is_the_regular_encode(B):
    require_gpu()
    rng = np.random.default_rng(31 + B)
    for n in (0, 1000, 16 * 65536, 16 * 65536 - 3):
        x = wl.mixed_small(rng, n)
        cache = wl.perturbed_cache(rng, x, 0.02) if B else None
        say(f"spec encode small n={n} B={B}")
        _check(x, B, cache, 255)


@pytest.mark.parametrize("B", [0, 256])
def test_spec_encode_after_waits_that_give_up(B):
    """With the wait bound at one poll the speculative write gives up and the
    two-pass kernels run; their waits may give up too.  Either the stream is
    the oracle's, or the call ends in the regular encode's failure state;
    after the documented recovery the next call is the oracle's again."""
    require_gpu()
    rng = np.random.default_rng(55 + B)
    n = 200 * 65536 + 3001
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    prev = exps(x).copy()
    prev[rng.random(n) < 0.001] ^= 1
    right = oracle.choose_e0(x)
    cap = ciera.ciera_max_encoded_size(n, B) if B else ciera.zip3_max_encoded_size(n)
    wsz = ciera.ciera_workspace_size(n, B) if B else ciera.zip3_workspace_size(n)
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    cache = torch.from_numpy(prev).cuda() if B else None
    hint = torch.tensor([right], dtype=torch.uint8, device="cuda")

    def call():
        if B:
            ciera.ciera_encode_spec(xd, B, cache, hint, out, ws, size)
        else:
            ciera.zip3_encode_spec(xd, hint, out, ws, size)
        torch.cuda.synchronize()
        return ciera.ciera_read_error(ws)

    old = ciera.ciera_set_wait_limit(1)
    try:
        say(f"spec encode with the wait bound at 1 poll, B={B}")
        st = call()
    finally:
        ciera.ciera_set_wait_limit(old)
    assert st in (0, ciera.STATUS_CODES["CIERA_ERR_INTERNAL"]), st
    zero = np.zeros(n, dtype=np.uint8)
    if st == 0:
        want, _ = oracle.encode(x, B, prev.copy() if B else None)
        assert out[:int(size.item())].cpu().numpy().tobytes() == want.tobytes()
    else:
        assert int(size.item()) == 0
        assert not out[:8].cpu().numpy().any(), "the header's first word still passes for a stream"
    if B:
        assert np.array_equal(cache.cpu().numpy(), exps(x))
        cache.zero_()  # recovery: a full resend
    size.fill_(-1)
    assert call() == 0
    want, _ = oracle.encode(x, B, zero.copy() if B else None)
    got = out[:int(size.item())].cpu().numpy()
    assert got.tobytes() == want.tobytes()
    check_roundtrip(got, x, B, zero.copy() if B else None)


def test_codec_encode_spec_equals_encode():
    """Codec objects: after a full encode, encode_spec takes its hint from
    byte 7 of the previous stream in the same output buffer and writes what
    the oracle (and so encode) writes, over iterations whose window stays and
    one whose window moves."""
    from lossless_bf16_tensor_exp_amd.codec import CieraCodec, Zip3Codec
    rng = np.random.default_rng(45)
    n = 3 * 65536 + 999
    xs = [wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))]
    for scale in (1.0, 1.0, 16.0):  # the last step moves the window
        x = wl.f32_to_bf16(wl.bf16_to_f32(xs[-1]) * np.float32(scale))
        wl.flip(x, rng.choice(n, size=3000, replace=False))
        xs.append(x)
    dev = [torch.from_numpy(x.view(np.int16)).cuda() for x in xs]
    say(f"codec encode_spec n={n}")
    z = Zip3Codec(n)
    z.encode(dev[0])
    for x, d in zip(xs[1:], dev[1:]):
        z.encode_spec(d)
        torch.cuda.synchronize()
        assert z.error() == 0
        o, _ = oracle.encode(x, 0, None)
        assert z.out[:z.nbytes()].cpu().numpy().tobytes() == o.tobytes()
    c = CieraCodec(n, 256)
    cache = np.zeros(n, np.uint8)
    c.encode(dev[0])
    oracle.encode(xs[0], 256, cache)
    for x, d in zip(xs[1:], dev[1:]):
        c.encode_spec(d)
        torch.cuda.synchronize()
        assert c.error() == 0
        o, _ = oracle.encode(x, 256, cache)
        assert c.out[:c.nbytes()].cpu().numpy().tobytes() == o.tobytes()
        assert np.array_equal(c.send_cache[:n].cpu().numpy(), cache)
