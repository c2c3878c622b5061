"""GPU parity of the single-read encode (window base given in device memory,
no variance pass): its stream must equal the oracle's at that window base,
byte for byte, and decode back to the input."""
import numpy as np
import pytest

import oracle
from gpu_util import (check_encode_e0, check_roundtrip, gpu_encode, gpu_encode_e0, require_gpu, say, torch)
from lossless_bf16_tensor_exp_amd import workloads as wl

pytestmark = pytest.mark.gpu

SMALL_N = [0, 1, 7, 8, 9, 63, 64, 65, 1000, 65535, 65536, 65537, 3 * 65536 + 12345, 16384, 16385, 49152 + 3]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n", SMALL_N)
def test_single_read_small(n):
    say(f"single-read n={n}")
    rng = np.random.default_rng(3000 + n)
    x = wl.mixed_small(rng, n)
    for e0 in (oracle.choose_e0(x), 0, 120, 249):
        s = check_encode_e0(x, e0)
        check_roundtrip(s, x)


def test_single_read_many_chunks():
    # 300 chunks: the look-back spans several rounds of 64 predecessors
    rng = np.random.default_rng(31)
    n = 300 * 65536 - 999
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.01))
    for e0 in (oracle.choose_e0(x), 110):
        s = check_encode_e0(x, e0)
    check_roundtrip(s, x)


def test_single_read_window_from_previous_stream():
    # the window base of iteration t is byte 7 of iteration t-1's stream,
    # read on the device
    rng = np.random.default_rng(32)
    n = 5 * 65536 + 77
    x0 = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    x1 = x0.copy()
    wl.flip(x1, rng.choice(n, size=4000, replace=False))
    s0, _ = gpu_encode(x0)
    prev = torch.from_numpy(s0).cuda()
    g, st = gpu_encode_e0(x1, prev, 7)
    assert st == 0
    o, ost = oracle.encode(x1, 0, None, int(s0[7]))
    assert g.tobytes() == o.tobytes()
    assert ost["E0"] == int(s0[7])
    check_roundtrip(g, x1)


def test_single_read_rejects_bad_window_base():
    from gpu_util import CANARY
    x = np.arange(70000, dtype=np.uint16)
    for n in (70000, 0):
        for bad in (250, 255):
            src = torch.tensor([bad], dtype=torch.uint8, device="cuda")
            g, st = gpu_encode_e0(x[:n], src)
            assert g is None and st == 1
            # only the first header word is written, and its E0 byte keeps the
            # bad value: a decoder rejects it, and so does a next single-read
            # encode that takes its window base from byte 7
            buf, size, st = gpu_encode_e0(x[:n], src, raw=True)
            assert st == 1 and size == 0
            assert buf[:8].tolist() == [0] * 7 + [bad]
            assert (buf[8:] == CANARY).all(), "bytes written past the first header word"
            chained = torch.from_numpy(buf[:16].copy()).cuda()
            g, st = gpu_encode_e0(x[:n], chained, e0_offset=7)
            assert g is None and st == 1


def test_single_read_deterministic():
    rng = np.random.default_rng(33)
    x = wl.f32_to_bf16(rng.standard_normal(3_000_000, dtype=np.float32))
    src = torch.tensor([oracle.choose_e0(x)], dtype=torch.uint8, device="cuda")
    a, _ = gpu_encode_e0(x, src)
    b, _ = gpu_encode_e0(x, src)
    assert a.tobytes() == b.tobytes()


def test_single_read_workload2():
    (g,) = wl.workload2()["iters"]
    say(f"single-read workload2 n={g.size}")
    s = check_encode_e0(g, 112)
    check_roundtrip(s, g)


# ---------------------------------------------------------------- ciera mode
from gpu_util import check_encode_e0_ciera, exps, gpu_encode_e0_ciera  # noqa: E402

CIERA_B = [64, 256, 512, 1024, 4096, 16384, 32768, 65536]


@pytest.mark.parametrize("B", CIERA_B)
@pytest.mark.parametrize("n", SMALL_N)
def test_single_read_ciera_small(n, B):
    say(f"single-read ciera n={n} B={B}")
    rng = np.random.default_rng(5000 + n + B)
    x = wl.mixed_small(rng, n)
    cache = wl.perturbed_cache(rng, x, 0.01)
    for e0 in (oracle.choose_e0(x), 120):
        s = check_encode_e0_ciera(x, B, cache, e0)
    recv = cache.copy()
    check_roundtrip(s, x, B, recv)


@pytest.mark.parametrize("B", [64, 1024, 32768])
def test_single_read_ciera_unchanged_and_all_changed(B):
    rng = np.random.default_rng(B + 1)
    n = 2 * 65536 + 5000
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))
    e0 = oracle.choose_e0(x)
    s = check_encode_e0_ciera(x, B, exps(x), e0)          # nothing changed: no planes, no escapes
    check_roundtrip(s, x, B, exps(x))
    s = check_encode_e0_ciera(x, B, np.zeros(n, np.uint8), e0)  # every block changed
    check_roundtrip(s, x, B, np.zeros(n, np.uint8))


@pytest.mark.parametrize("B", [64, 4096])
def test_single_read_ciera_many_chunks(B):
    # 300 chunks: the look-back spans several rounds of 64 predecessors,
    # each predecessor's size from its parts' words
    rng = np.random.default_rng(41 + B)
    n = 300 * 65536 - 999
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.01))
    cache = wl.perturbed_cache(rng, x, 0.002)
    s = check_encode_e0_ciera(x, B, cache, oracle.choose_e0(x))
    check_roundtrip(s, x, B, cache.copy())


def test_single_read_ciera_rejects_bad_window_base():
    rng = np.random.default_rng(42)
    x = wl.mixed_small(rng, 70000)
    cache = wl.perturbed_cache(rng, x, 0.05)
    for bad in (250, 255):
        g, st, gc = gpu_encode_e0_ciera(x, 256, cache.copy(), torch.tensor([bad], dtype=torch.uint8, device="cuda"))
        assert g is None and st == 1
        assert np.array_equal(gc, cache), "the cache changed although nothing was encoded"


def test_single_read_ciera_workload3():
    d = wl.workload3()
    x0, x1 = d["iters"]
    say(f"single-read ciera workload3 n={x1.size}")
    s = check_encode_e0_ciera(x1, 64, exps(x0), 116)
    check_roundtrip(s, x1, 64, exps(x0))


def test_codec_encode_e0_takes_the_previous_window():
    """Codec objects: after a full encode, encode_e0 takes the window base
    from byte 7 of the previous stream in the same output buffer."""
    from lossless_bf16_tensor_exp_amd.codec import CieraCodec, Zip3Codec
    rng = np.random.default_rng(44)
    n = 3 * 65536 + 999
    xs = [wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02))]
    for _ in range(2):
        x = xs[-1].copy()
        wl.flip(x, rng.choice(n, size=3000, replace=False))
        xs.append(x)
    dev = [torch.from_numpy(x.view(np.int16)).cuda() for x in xs]
    z = Zip3Codec(n)
    z.encode(dev[0])
    torch.cuda.synchronize()
    e0 = int(z.out[7].item())
    for x, d in zip(xs[1:], dev[1:]):
        z.encode_e0(d)
        torch.cuda.synchronize()
        assert z.error() == 0
        o, st = oracle.encode(x, 0, None, e0)
        assert z.out[:z.nbytes()].cpu().numpy().tobytes() == o.tobytes() and st["E0"] == e0
    c = CieraCodec(n, 256)
    cache = np.zeros(n, np.uint8)
    c.encode(dev[0])
    oracle.encode(xs[0], 256, cache)
    torch.cuda.synchronize()
    e0 = int(c.out[7].item())
    for x, d in zip(xs[1:], dev[1:]):
        c.encode_e0(d)
        torch.cuda.synchronize()
        assert c.error() == 0
        o, _ = oracle.encode(x, 256, cache, e0)
        assert c.out[:c.nbytes()].cpu().numpy().tobytes() == o.tobytes()
        assert np.array_equal(c.send_cache[:n].cpu().numpy(), cache)
