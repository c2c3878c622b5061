"""Calls on two HIP streams at once, each with its own workspace and
buffers: every encode of a batch is enqueued before any finishes (3-bit
two-pass, single-read, speculative (right and wrong hint), hash sender and
rANS encodes, whose kernels wait on other workgroups of their own launch),
then every decode.  Each stream
and each decoded tensor must equal what the same call gives alone on the
default stream; those single calls are checked against the oracle by the
other GPU tests."""
import numpy as np
import pytest

from gpu_util import require_gpu, say
from lossless_bf16_tensor_exp_amd import workloads as wl

torch = pytest.importorskip("torch")
import lossless_bf16_tensor_exp_amd as ciera  # noqa: E402

pytestmark = pytest.mark.gpu

N = 3_000_000 + 4099  # 46 chunks, the last one partial


def _inputs(seed):
    rng = np.random.default_rng(seed)
    x0 = wl.f32_to_bf16(rng.standard_normal(N, dtype=np.float32) * np.float32(0.02))
    x1 = x0.copy()
    x1[rng.random(N) < 0.002] ^= np.uint16(0x0080)  # exponent flips: some blocks change
    return x0, x1


class Job:
    """One encode (and later its decode) with buffers of its own."""

    def __init__(self, kind, B, x0, x1):
        self.kind, self.B = kind, B
        dev = "cuda"
        self.x = torch.from_numpy(x1.view(np.int16)).to(dev)
        n = x1.size
        rans = kind.startswith("rans")
        if rans:
            cap, wsz = ciera.rans_max_encoded_size(n, B), ciera.rans_workspace_size(n, B)
        elif B:
            cap, wsz = ciera.ciera_max_encoded_size(n, B), ciera.ciera_workspace_size(n, B)
        else:
            cap, wsz = ciera.zip3_max_encoded_size(n), ciera.zip3_workspace_size(n)
        self.cap = cap
        self.out = torch.zeros(cap, dtype=torch.uint8, device=dev)
        self.ws = torch.zeros(wsz, dtype=torch.uint8, device=dev)
        self.dws = torch.zeros(wsz, dtype=torch.uint8, device=dev)
        self.size = torch.zeros(1, dtype=torch.int64, device=dev)
        self.y = torch.zeros(n, dtype=torch.int16, device=dev)
        e_prev = torch.from_numpy(((x0 >> 7) & 0xFF).astype(np.uint8)).to(dev)
        self.send = e_prev.clone()
        self.recv = e_prev.clone()
        if kind == "hashed":
            self.hcache = torch.zeros(ciera.ciera_hash_cache_size(n, B), dtype=torch.uint8, device=dev)
            # the hashes of x0's exponents, from one hashed encode of x0
            x0d = torch.from_numpy(x0.view(np.int16)).to(dev)
            ciera.ciera_encode_hashed(x0d, B, self.hcache, self.out, self.ws, self.size)
        if kind == "single" or kind.startswith("spec"):
            # the window base from a full encode of the same tensor (a wrong
            # hint for "spec_miss": one binade up)
            self.e0 = torch.zeros(16, dtype=torch.uint8, device=dev)
            ciera.zip3_encode(self.x, self.out, self.ws, self.size)
            torch.cuda.synchronize()
            self.e0.copy_(self.out[:16])
            if kind == "spec_miss":
                self.e0[7] += 1
        torch.cuda.synchronize()
        self.hcache0 = self.hcache.clone() if kind == "hashed" else None

    def reset(self):
        self.send.copy_(self.recv)
        if self.hcache0 is not None:
            self.hcache.copy_(self.hcache0)

    def encode(self, stream):
        k, B = self.kind, self.B
        if k == "zip3":
            ciera.zip3_encode(self.x, self.out, self.ws, self.size, stream=stream)
        elif k == "ciera":
            ciera.ciera_encode(self.x, B, self.send, self.out, self.ws, self.size, stream=stream)
        elif k == "single":
            ciera.zip3_encode_e0(self.x, self.e0, self.out, self.ws, self.size, e0_offset=7, stream=stream)
        elif k == "hashed":
            ciera.ciera_encode_hashed(self.x, B, self.hcache, self.out, self.ws, self.size, stream=stream)
        elif k == "spec" and B:
            ciera.ciera_encode_spec(self.x, B, self.send, self.e0, self.out, self.ws, self.size, hint_offset=7,
                                    stream=stream)
        elif k in ("spec", "spec_miss"):
            ciera.zip3_encode_spec(self.x, self.e0, self.out, self.ws, self.size, hint_offset=7, stream=stream)
        elif k == "rans_zip3":
            ciera.zip3_encode_rans(self.x, self.out, self.ws, self.size, stream=stream)
        elif k == "rans_ciera":
            ciera.ciera_encode_rans(self.x, B, self.send, self.out, self.ws, self.size, stream=stream)

    def decode(self, stream, sz):
        k, B = self.kind, self.B
        if k in ("zip3", "single", "spec_miss") or (k == "spec" and not B):
            ciera.zip3_decode(self.out, sz, self.y, self.dws, stream=stream)
        elif k in ("ciera", "hashed", "spec"):
            ciera.ciera_decode(self.out, sz, self.y, B, self.recv, self.dws, stream=stream)
        elif k == "rans_zip3":
            ciera.zip3_decode_rans(self.out, sz, self.y, self.dws, stream=stream)
        elif k == "rans_ciera":
            ciera.ciera_decode_rans(self.out, sz, self.y, B, self.recv, self.dws, stream=stream)


KINDS = [("zip3", 0), ("ciera", 64), ("single", 0), ("hashed", 256), ("rans_zip3", 0), ("rans_ciera", 128),
         ("ciera", 1024), ("zip3", 0), ("spec", 256), ("spec_miss", 0)]


def test_two_streams_overlapping_calls():
    require_gpu()
    jobs = []
    for i, (kind, B) in enumerate(KINDS):
        x0, x1 = _inputs(100 + i)
        jobs.append(Job(kind, B, x0, x1))
    # alone, on the default stream: the expected streams
    want = []
    for j in jobs:
        j.reset()
        j.encode(None)
        torch.cuda.synchronize()
        assert ciera.ciera_read_error(j.ws) == 0, j.kind
        sz = int(j.size.item())
        want.append(j.out[:sz].clone())
    # every encode enqueued on one of two streams before any is waited for
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for j in jobs:
        j.reset()
        j.out.zero_()
    torch.cuda.synchronize()
    for i, j in enumerate(jobs):
        j.encode(streams[i % 2])
    torch.cuda.synchronize()
    sizes = []
    for j, w in zip(jobs, want):
        assert ciera.ciera_read_error(j.ws) == 0, j.kind
        sz = int(j.size.item())
        say(f"{j.kind} B={j.B}: {sz} bytes")
        assert sz == w.numel() and torch.equal(j.out[:sz], w), f"{j.kind} B={j.B}: stream differs under concurrency"
        sizes.append(sz)
    # then every decode the same way (receiver caches start at x0's exponents)
    for i, j in enumerate(jobs):
        j.decode(streams[i % 2], sizes[i])
    torch.cuda.synchronize()
    for j in jobs:
        assert ciera.ciera_read_error(j.dws) == 0, j.kind
        assert torch.equal(j.y, j.x), f"{j.kind} B={j.B}: round trip failed under concurrency"
        if j.B:
            assert torch.equal(j.recv, ((j.x.to(torch.int32) >> 7) & 0xFF).to(torch.uint8)), j.kind
