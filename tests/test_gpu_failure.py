"""Failure and contention paths of the encodes that wait on other
workgroups, all driven from the host so that every kernel ends normally.

- A lowered wait bound (the ciera_set_wait_limit test hook) makes the waits
  give up: the encode must report CIERA_ERR_INTERNAL and leave the state its
  header documents (the 3-bit two-pass encode: *out_size 0, header cleared,
  a decoder rejects the stream); after the documented recovery (zero the
  sender's and the receiver's caches) the next encode equals the oracle's
  from zero caches and decodes back.
- An encode enqueued while a long elementwise workload runs on a second
  stream completes with status 0 and the oracle's bytes: no workgroup waits
  on one that is dispatched after it.
"""
import numpy as np
import pytest

import oracle
from gpu_util import check_roundtrip, exps, require_gpu, say
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")
import lossless_bf16_tensor_exp_amd as ciera  # noqa: E402

pytestmark = pytest.mark.gpu

N = 200 * 65536 + 3001  # 201 chunks: the planner runs 13 groups


def _input(seed):
    rng = np.random.default_rng(seed)
    x = wl.f32_to_bf16(rng.standard_normal(N, dtype=np.float32) * np.float32(0.02))
    prev = exps(x).copy()
    prev[rng.random(N) < 0.001] ^= 1
    return x, prev


def _encode(kind, xd, n, B, cache, out, ws, size, e0_src=None):
    if kind == "zip3":
        ciera.zip3_encode(xd, out, ws, size)
    elif kind == "ciera":
        ciera.ciera_encode(xd, B, cache, out, ws, size)
    elif kind == "single":
        ciera.ciera_encode_e0(xd, B, cache, e0_src, out, ws, size)
    elif kind == "rans":
        ciera.ciera_encode_rans(xd, B, cache, out, ws, size)
    else:
        raise ValueError(kind)


@pytest.mark.parametrize("kind", ["zip3", "ciera", "single", "rans"])
def test_wait_failure_is_reported_and_recoverable(kind):
    require_gpu()
    B = 0 if kind == "zip3" else 256
    x, prev = _input(1)
    n = x.size
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    if kind == "rans":
        cap, wsz = ciera.rans_max_encoded_size(n, B), ciera.rans_workspace_size(n, B)
    elif B:
        cap, wsz = ciera.ciera_max_encoded_size(n, B), ciera.ciera_workspace_size(n, B)
    else:
        cap, wsz = ciera.zip3_max_encoded_size(n), ciera.zip3_workspace_size(n)
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    ws = torch.zeros(wsz, dtype=torch.uint8, device="cuda")
    size = torch.full((1,), -1, dtype=torch.int64, device="cuda")
    cache = torch.from_numpy(prev).cuda() if B else None
    e0_src = torch.tensor([oracle.choose_e0(x)], dtype=torch.uint8, device="cuda")
    failed = False
    old = ciera.ciera_set_wait_limit(1)
    try:
        for attempt in range(3):
            if B:
                cache.copy_(torch.from_numpy(prev))
            size.fill_(-1)
            say(f"failure path {kind}: attempt {attempt} with the wait bound at 1 poll")
            _encode(kind, xd, n, B, cache, out, ws, size, e0_src)
            torch.cuda.synchronize()
            st = ciera.ciera_read_error(ws)
            assert st in (0, ciera.STATUS_CODES["CIERA_ERR_INTERNAL"]), st
            if st:
                failed = True
                break
    finally:
        ciera.ciera_set_wait_limit(old)
    assert ciera.ciera_set_wait_limit(0) == old  # the default bound is back
    assert failed, "no wait gave up at a bound of one poll"
    if kind in ("zip3", "ciera"):
        assert int(size.item()) == 0
        assert not out[:8].cpu().numpy().any(), "the header's first word still passes for a stream"
        # a decoder rejects what is left
        y = torch.empty(n, dtype=torch.int16, device="cuda")
        dws = torch.empty(wsz, dtype=torch.uint8, device="cuda")
        if B:
            ciera.ciera_decode(out, cap, y, B, torch.zeros(n, dtype=torch.uint8, device="cuda"), dws)
        else:
            ciera.zip3_decode(out, cap, y, dws)
        assert ciera.ciera_read_error(dws) == ciera.STATUS_CODES["CIERA_ERR_FORMAT"]
    # recovery: both caches zeroed, the next encode is a full resend
    if B:
        cache.zero_()
    size.fill_(-1)
    _encode(kind, xd, n, B, cache, out, ws, size, e0_src)
    torch.cuda.synchronize()
    assert ciera.ciera_read_error(ws) == 0
    sz = int(size.item())
    got = out[:sz].cpu().numpy()
    zero = np.zeros(n, dtype=np.uint8)
    if kind == "rans":
        want, _ = oracle.encode_rans(x, B, zero.copy())
    elif kind == "single":
        want, _ = oracle.encode(x, B, zero.copy(), int(e0_src.item()))
    else:
        want, _ = oracle.encode(x, B, zero.copy() if B else None)
    assert got.tobytes() == want.tobytes()
    if B:
        assert np.array_equal(cache.cpu().numpy(), exps(x))
    if kind != "rans":
        check_roundtrip(got, x, B, zero.copy() if B else None)


def test_encode_completes_beside_a_long_workload_on_another_stream():
    """A long elementwise workload (many launches over 1 GiB) is enqueued
    on a second stream, then encodes on the first; each must end with
    status 0 and the oracle's bytes."""
    require_gpu()
    x, prev = _input(2)
    n = x.size
    B = 512
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    big = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    want_z, _ = oracle.encode(x)
    want_c, _ = oracle.encode(x, B, prev.copy())
    s_busy = torch.cuda.Stream()
    s_enc = torch.cuda.Stream()
    cap, wsz = ciera.ciera_max_encoded_size(n, B), ciera.ciera_workspace_size(n, B)
    torch.cuda.synchronize()
    for rep in range(3):
        say(f"encode beside a busy stream, rep {rep}")
        outs = [torch.zeros(cap, dtype=torch.uint8, device="cuda") for _ in range(2)]
        wss = [torch.zeros(wsz, dtype=torch.uint8, device="cuda") for _ in range(2)]
        sizes = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in range(2)]
        cache = torch.from_numpy(prev).cuda()
        torch.cuda.synchronize()
        with torch.cuda.stream(s_busy):
            for _ in range(40):
                big.mul_(1.0000001)
        ciera.zip3_encode(xd, outs[0], wss[0], sizes[0], stream=s_enc)
        ciera.ciera_encode(xd, B, cache, outs[1], wss[1], sizes[1], stream=s_enc)
        torch.cuda.synchronize()
        for k, want in enumerate((want_z, want_c)):
            assert ciera.ciera_read_error(wss[k]) == 0
            got = outs[k][: int(sizes[k].item())].cpu().numpy()
            assert got.tobytes() == want.tobytes(), (rep, k)
        assert np.array_equal(cache.cpu().numpy(), exps(x))
