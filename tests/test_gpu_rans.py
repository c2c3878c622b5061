"""GPU parity of the rANS modes (zip3 + rANS, ciera + rANS): streams byte for
byte equal to the oracle's, decode returns the input bit for bit, caches
match, canary guards intact; malformed streams are rejected.  A chunk's
four parts are coded by four waves against the chunk's one table; payloads
beyond the decoder's 32 KB LDS stage (all 65536 patterns, random bits) take
the HBM word path."""
import numpy as np
import pytest

import oracle
from gpu_util import check_rans, exps, gpu_decode_rans, gpu_encode_rans, require_gpu, say
from lossless_bf16_tensor_exp_amd import workloads as wl

pytestmark = pytest.mark.gpu

SMALL_N = [0, 1, 7, 8, 9, 63, 64, 65, 1000, 16383, 16384, 16385, 65535, 65536, 65537, 3 * 65536 + 12345]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n", SMALL_N)
def test_zip3_rans_small(n):
    say(f"zip3 rans n={n}")
    rng = np.random.default_rng(3000 + n)
    for _ in range(2):
        check_rans(wl.mixed_small(rng, n))


@pytest.mark.parametrize("B", [64, 256, 512, 1024, 4096, 32768, 65536])
@pytest.mark.parametrize("n", SMALL_N)
def test_ciera_rans_small(n, B):
    say(f"ciera rans n={n} B={B}")
    rng = np.random.default_rng(4000 + n + B)
    x = wl.mixed_small(rng, n)
    check_rans(x, B, wl.perturbed_cache(rng, x, 0.01))
    x2 = x.copy()
    if n:
        wl.flip(x2, rng.choice(n, size=max(1, n // 300), replace=False))
    check_rans(x2, B, exps(x))


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_rans_all_patterns(order):
    x = wl.all_bf16_patterns()
    if order == "shuffled":
        x = x[np.random.default_rng(8).permutation(x.size)]
    check_rans(x)
    check_rans(x, 512, np.zeros(x.size, dtype=np.uint8))


@pytest.mark.parametrize("sigma", [1e-3, 0.02, 1.0])
def test_rans_gaussian_many_chunks(sigma):
    rng = np.random.default_rng(int(sigma * 1000) + 5)
    x = wl.normal_bf16(rng, 37 * 65536 - 999, sigma)
    check_rans(x)


def test_rans_gradient_64M():
    d = wl.workload2()
    x = d["iters"][0]
    say(f"rans workload2 n={x.size}")
    s = check_rans(x)
    t, _ = oracle.encode(x)
    say(f"  rANS ratio {2 * x.size / s.size:.4f}, 3-bit ratio {2 * x.size / t.size:.4f}")
    assert s.size < t.size


def test_rans_olmoe_shard_B64():
    d = wl.workload3()
    x0, x1 = d["iters"]
    say(f"rans workload3 n={x0.size}")
    s = check_rans(x1, 64, exps(x0))
    say(f"  rANS ratio {2 * x1.size / s.size:.4f}")


def test_rans_decode_rejects_corruption():
    rng = np.random.default_rng(6)
    x = wl.normal_bf16(rng, 65536, 0.02)
    s, _ = gpu_encode_rans(x)
    a = int(s[128:136].view(np.uint64)[0])
    nw = [int(v) for v in s[a + 4:a + 12].view(np.uint16)]
    lo, hi = int(s[a]), int(s[a + 1])
    words = a + 12 + 2 * (hi - lo + 1)        # part 0's stream
    words3 = words + 2 * sum(nw[:3])          # part 3's stream
    cases = {
        "mode byte": (6, 0),
        "version": (4, 1),
        "part 0 word count": (a + 4, (nw[0] + 1) & 0xFF),
        "part 2 word count": (a + 8, (nw[2] - 1) & 0xFF),
        "frequency": (a + 12, s[a + 12] ^ 1),
        "renormalisation word": (words + 256 + 20, s[words + 256 + 20] ^ 0x10),
        "final state": (words + 3, s[words + 3] ^ 0x80),
        "part 3 final state": (words3 + 130, s[words3 + 130] ^ 0x80),
        "chunk table": (136, s[136] ^ 0x40),
    }
    for name, (at, val) in cases.items():
        t = s.copy()
        t[at] = val
        with pytest.raises(oracle.OracleError):
            oracle.decode_rans(t, x.size)
        _, _, st = gpu_decode_rans(t, x.size)
        assert st == 5, f"{name}: status {st}"
    y, _, st = gpu_decode_rans(s, x.size)
    assert st == 0 and np.array_equal(y, x)


def test_rans_decode_rejects_moved_part_boundary():
    """Word counts that keep the payload length but move a boundary between
    two parts' streams (one part then runs into the next one's words), and a
    corruption in a later chunk of several, are rejected without writes past
    the outputs (the canary guards)."""
    rng = np.random.default_rng(7)
    x = wl.normal_bf16(rng, 3 * 65536 + 4321, 0.02)
    s, _ = gpu_encode_rans(x)
    table = s[128:128 + 8 * 5].view(np.uint64)
    cases = {}
    for c in (0, 2):
        a = int(table[c])
        nw = [int(v) for v in s[a + 4:a + 12].view(np.uint16)]
        for h in range(3):
            if nw[h + 1]:
                t = s.copy()
                t[a + 4:a + 12] = np.array(nw[:h] + [nw[h] + 1, nw[h + 1] - 1] + nw[h + 2:], np.uint16).view(np.uint8)
                cases[f"chunk {c}: boundary between parts {h} and {h + 1}"] = t
        t = s.copy()
        t[a + 4:a + 6] = np.array([0xFFFF], np.uint16).view(np.uint8)
        cases[f"chunk {c}: part 0 word count 65535"] = t
    for name, t in cases.items():
        with pytest.raises(oracle.OracleError):
            oracle.decode_rans(t, x.size)
        _, _, st = gpu_decode_rans(t, x.size)
        assert st == 5, f"{name}: status {st}"
    y, _, st = gpu_decode_rans(s, x.size)
    assert st == 0 and np.array_equal(y, x)
