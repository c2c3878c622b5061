"""GPU parity: the HIP library, called through its C ABI, against the CPU oracle.

Streams must equal the oracle's byte for byte (header, table, every section
and its zero padding), decode must return the input bit for bit, and both
exponent caches must match.  Output buffers carry canary guards on both sides
and past the stream's end.
"""
import numpy as np
import pytest

import oracle
from gpu_util import (check_encode, check_roundtrip, ciera, exps, gpu_decode, gpu_encode, require_gpu, say,
                      torch)
from lossless_bf16_tensor_exp_amd import workloads as wl

pytestmark = pytest.mark.gpu

SMALL_N = [0, 1, 7, 8, 9, 63, 64, 65, 1000, 65535, 65536, 65537, 3 * 65536 + 12345]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("n", SMALL_N)
def test_zip3_small(n):
    say(f"zip3 small n={n}")
    rng = np.random.default_rng(1000 + n)
    for _ in range(3):
        x = wl.mixed_small(rng, n)
        s, _ = check_encode(x)
        check_roundtrip(s, x)


@pytest.mark.parametrize("B", [64, 256, 4096, 65536])
@pytest.mark.parametrize("n", SMALL_N)
def test_ciera_small(n, B):
    say(f"ciera small n={n} B={B}")
    rng = np.random.default_rng(2000 + n + B)
    x = wl.mixed_small(rng, n)
    send = wl.perturbed_cache(rng, x, 0.01)
    recv = send.copy()
    s, _ = check_encode(x, B, send)
    check_roundtrip(s, x, B, recv)
    # second iteration from the updated caches
    x2 = x.copy()
    if n:
        wl.flip(x2, rng.choice(n, size=max(1, n // 300), replace=False))
    s2, st = check_encode(x2, B, exps(x))
    check_roundtrip(s2, x2, B, exps(x))


@pytest.mark.parametrize("order", ["sorted", "reversed", "shuffled"])
def test_all_bf16_patterns(order):
    say(f"all patterns {order}")
    x = wl.all_bf16_patterns()
    if order == "reversed":
        x = x[::-1].copy()
    elif order == "shuffled":
        x = np.random.default_rng(5).permutation(x)
    s, _ = check_encode(x)
    check_roundtrip(s, x)
    for B in (64, 512):
        prev = np.zeros(x.size, dtype=np.uint8)
        s, _ = check_encode(x, B, prev)
        check_roundtrip(s, x, B, prev)


@pytest.mark.parametrize("e0", [0, 1, 116, 248, 249])
def test_forced_window(e0):
    say(f"forced window {e0}")
    rng = np.random.default_rng(e0)
    x = wl.mixed_small(rng, 150000)
    s, st = check_encode(x, 0, None, e0)
    assert st["E0"] == e0
    check_roundtrip(s, x)
    prev = wl.perturbed_cache(rng, x, 0.02)
    s, _ = check_encode(x, 128, prev, e0)
    check_roundtrip(s, x, 128, prev)


def test_constant_and_nonfinite_tensors():
    for val in (0x0000, 0x8000, 0x3F80, 0x7FC0, 0xFF80):
        x = np.full(70000, val, dtype=np.uint16)
        s, st = check_encode(x)
        assert st["E0"] == 0
        check_roundtrip(s, x)


def test_extreme_magnitudes():
    # variance near the top of the BF16 range clamps the window base at 249;
    # tiny tensors (subnormals, smallest normals) clamp it at 0
    rng = np.random.default_rng(12)
    big = np.where(rng.random(100000) < 0.5, 0x7F7F, 0xFF7F).astype(np.uint16)
    s, st = check_encode(big)
    assert st["E0"] == 249
    check_roundtrip(s, big)
    tiny = rng.integers(0, 0x0100, size=100000).astype(np.uint16) | (rng.integers(0, 2, 100000).astype(np.uint16) << 15)
    s, st = check_encode(tiny)
    assert st["E0"] == 0
    check_roundtrip(s, tiny)


@pytest.mark.parametrize("k", [-40, -11, 30])
def test_variance_on_a_window_threshold(k):
    """Tensors whose exact variance equals K0 4^k, or misses it by a part in
    about 2^130: the oracle (exact) and the GPU (FP64) may pick either
    adjacent window base only here, and the rest of the stream must equal
    the oracle's at the GPU's base (check_encode); every stream decodes."""
    from test_oracle_exact import _threshold_tensor
    s_ = min(40, k - 17 + 126)
    for delta in (-1, 0, 1):
        x = _threshold_tensor(k, delta, s_)  # 513 values: 64 units and a ragged tail
        s, st = check_encode(x)
        assert int(s[7]) in (126 + k, 127 + k)
        check_roundtrip(s, x)
        s, _ = check_encode(x, 64, np.zeros(x.size, np.uint8))
        check_roundtrip(s, x, 64, np.zeros(x.size, np.uint8))


def test_deterministic_and_stream_independent():
    rng = np.random.default_rng(77)
    x = wl.f32_to_bf16(rng.standard_normal(5_000_000, dtype=np.float32) * np.float32(0.02))
    a, _ = gpu_encode(x)
    b, _ = gpu_encode(x)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        c, _ = gpu_encode(x, stream=side)
    assert a.tobytes() == b.tobytes() == c.tobytes()


def test_decode_rejects_malformed_streams():
    rng = np.random.default_rng(9)
    n = 200000
    x = wl.f32_to_bf16(rng.standard_normal(n, dtype=np.float32))
    good, _ = gpu_encode(x)
    y, _, st = gpu_decode(good, n)
    assert st == 0 and np.array_equal(y, x)
    idx = 128 + 8 * 5  # four chunks: five table entries, then the escape index
    for off, val in [(0, 0x41), (4, 2), (6, 1), (7, 250), (8, 0x71), (22, 0), (24, 9), (33, 0xEE), (60, 1),
                     (128, 0x80), (136, 1), (144, 0x11), (idx, 1), (idx + 4, 0x7F), (idx + 10, 0xFF),
                     (idx + 30, 0x3F), (idx + 32, 1)]:
        bad = good.copy()
        assert bad[off] != val
        bad[off] = val
        _, _, st = gpu_decode(bad, n)
        assert st == 5, off
    _, _, st = gpu_decode(good, n, in_size=good.size - 128)
    assert st == 5
    _, _, st = gpu_decode(good, n + 1)
    assert st == 5
    # a zip3 stream offered to the ciera decoder
    _, _, st = gpu_decode(good, n, 64, np.zeros(n, np.uint8))
    assert st == 5


def test_host_side_argument_errors():
    xd = torch.zeros(1000, dtype=torch.int16, device="cuda")
    ws = torch.empty(ciera.ciera_workspace_size(1000, 64), dtype=torch.uint8, device="cuda")
    size = torch.zeros(1, dtype=torch.int64, device="cuda")
    cache = torch.zeros(1000, dtype=torch.uint8, device="cuda")
    small = torch.empty(100, dtype=torch.uint8, device="cuda")
    out = torch.empty(ciera.ciera_max_encoded_size(1000, 64), dtype=torch.uint8, device="cuda")
    with pytest.raises(ciera.CieraError) as e:
        ciera.zip3_encode(xd, small, ws, size)
    assert e.value.status == 2
    with pytest.raises(ciera.CieraError) as e:
        ciera.ciera_encode(xd, 100, cache, out, ws, size)
    assert e.value.status == 1
    with pytest.raises(ciera.CieraError) as e:
        ciera.zip3_encode(xd, out, ws[:16], size)
    assert e.value.status == 3
    with pytest.raises(ciera.CieraError) as e:
        ciera.zip3_encode(xd, out, ws, size, e0_override=250)
    assert e.value.status == 1
    with pytest.raises(ciera.CieraError) as e:
        ciera.zip3_encode(xd[1:], out, ws, size)  # misaligned input
    assert e.value.status == 1


# ---------------------------------------------------------------- workloads at full size
def test_workload1_shard_iteration():
    d = wl.workload1()
    x0, x1 = d["iters"]
    B = d["B"][0]
    say(f"workload1 n={x0.size} B={B}")
    zero = np.zeros(x0.size, dtype=np.uint8)
    s0, _ = check_encode(x0, B, zero)
    check_roundtrip(s0, x0, B, zero)
    s1, st = check_encode(x1, B, exps(x0))
    check_roundtrip(s1, x1, B, exps(x0))
    say(f"  E0={st['E0']} changed={st['changed_blocks']} esc={st['escapes']} ratio={2 * x1.size / s1.size:.3f}")


def test_workload2_gradient_zip3():
    d = wl.workload2()
    (g,) = d["iters"]
    say(f"workload2 n={g.size}")
    s, st = check_encode(g)
    check_roundtrip(s, g)
    say(f"  E0={st['E0']} esc={st['escapes']} ratio={2 * g.size / s.size:.3f}")
    assert st["E0"] == 112


def test_workload3_layer_block_sweep():
    d = wl.workload3()
    x0, x1 = d["iters"]
    say(f"workload3 n={x0.size}")
    for B in d["B"]:
        s, st = check_encode(x1, B, exps(x0))
        check_roundtrip(s, x1, B, exps(x0))
        nb = -(-x1.size // B)
        say(f"  B={B} reuse={1 - st['changed_blocks'] / nb:.3f} ratio={2 * x1.size / s.size:.3f}")


def test_workload4_ten_iteration_chain():
    d = wl.workload4()
    it = d["iters"]
    B = d["B"][0]
    say(f"workload4 n={it[0].size} iterations={len(it) - 1}")
    send = np.zeros(it[0].size, dtype=np.uint8)
    recv = send.copy()
    for t, x in enumerate(it):
        s, st = check_encode(x, B, send)
        recv = check_roundtrip(s, x, B, recv)
        send = exps(x)
        say(f"  iter {t} changed={st['changed_blocks']} ratio={2 * x.size / s.size:.3f}")


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_workload5_stress_billion():
    d = wl.workload5()
    x0, x1 = d["iters"]
    B = d["B"][0]
    say(f"workload5 n={x0.size} B={B}")
    # x0 from zero caches on the GPU only (the cache it leaves is checked
    # against E(x0)); x1 against that cache is the full oracle comparison.
    _, c = gpu_encode(x0, B, np.zeros(x0.size, dtype=np.uint8))
    assert np.array_equal(c, exps(x0))
    del c
    s, st = check_encode(x1, B, exps(x0))
    say(f"  E0={st['E0']} changed={st['changed_blocks']} esc={st['escapes']} ratio={2 * x1.size / s.size:.3f}")
    check_roundtrip(s, x1, B, exps(x0))
