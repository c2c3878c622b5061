"""GPU parity of the planning step at many chunk counts and workgroup shapes.

The planner splits the chunks over up to 256 workgroups (at least 16 chunks
each), every group taking its chunks 256 at a time.  ``plan_groups`` caps the
group count, so that small inputs reach the shapes large ones take: several
rounds per group (register path) and more than eight rounds (the chunk table
holds the group-relative offsets between its two passes).  Every stream must
equal the oracle's byte for byte, and the stream does not depend on the
shape.
"""
import numpy as np
import pytest

from gpu_util import check_encode, check_roundtrip, gpu_encode, require_gpu, say
from lossless_bf16_tensor_exp_amd import workloads as wl

pytestmark = pytest.mark.gpu
C = wl.CHUNK


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def varied(n, seed):
    """BF16 values whose scale changes from chunk to chunk, so chunk sizes
    and escape counts vary: each chunk is a random window of one 8M-value
    N(0, 1e-3) draw times 2^k, k in -3..3 (an exact shift of the exponent
    field: every value of the pool is a normal number far from the ends of
    the exponent range).  Three chunks hold a mix of every BF16 class."""
    rng = np.random.default_rng(seed)
    nchunks = -(-n // C)
    pool = wl.normal_bf16(rng, 1 << 23, 1e-3)
    e = (pool >> 7) & 0xFF
    pool[(e < 8) | (e > 240)] = 0x3A83  # the draw's rare exact zeros: about 1e-3 instead
    x = np.empty(n, dtype=np.uint16)
    offs = rng.integers(0, pool.size - C, size=nchunks)
    shifts = rng.integers(-3, 4, size=nchunks)
    for c in range(nchunks):
        lo, hi = c * C, min(n, (c + 1) * C)
        x[lo:hi] = pool[offs[c]:offs[c] + hi - lo] + np.uint16((int(shifts[c]) << 7) & 0xFFFF)
    for c in rng.choice(nchunks, size=min(nchunks, 3), replace=False):
        lo, hi = c * C, min(n, (c + 1) * C)
        x[lo:hi] = wl.mixed_small(rng, hi - lo)
    return x


@pytest.mark.parametrize("nchunks,tail", [(17, 0), (33, 100), (40, 65535)])
@pytest.mark.parametrize("groups", [0, 1, 2, 3])
def test_plan_shapes_small(nchunks, tail, groups):
    n = nchunks * C - tail
    say(f"plan shapes n={n} groups={groups}")
    x = varied(n, 7 + nchunks)
    s, _ = check_encode(x, plan_groups=groups)
    check_roundtrip(s, x)


@pytest.mark.parametrize("B", [128, 32768])
def test_plan_shapes_ciera(B):
    n = 40 * C - 333
    say(f"plan shapes ciera n={n} B={B}")
    rng = np.random.default_rng(B)
    x = varied(n, 11)
    send = wl.perturbed_cache(rng, x, 0.002)
    recv = send.copy()
    for groups in (0, 1, 3):
        s, _ = check_encode(x, B, send.copy(), plan_groups=groups)
    check_roundtrip(s, x, B, recv)


def test_plan_register_rounds():
    """One group over 1,100 chunks: five rounds of 256 chunks each."""
    n = 1100 * C - 777
    say(f"plan register rounds n={n}")
    x = varied(n, 21)
    s, _ = check_encode(x, plan_groups=1)
    for groups in (0, 2, 5):
        g, _ = gpu_encode(x, plan_groups=groups)
        assert g.tobytes() == s.tobytes(), f"stream depends on the plan shape ({groups} groups)"
    check_roundtrip(s, x)


def test_plan_table_rounds():
    """One group over 2,305 chunks: ten rounds, more than the registers hold."""
    n = 2305 * C - 12345
    say(f"plan table rounds n={n}")
    x = varied(n, 22)
    s, _ = check_encode(x, plan_groups=1)
    check_roundtrip(s, x)


def test_plan_table_rounds_ciera():
    n = 2305 * C - 12345
    say(f"plan table rounds ciera n={n}")
    rng = np.random.default_rng(23)
    x = varied(n, 23)
    send = wl.perturbed_cache(rng, x, 0.001)
    s, _ = check_encode(x, 512, send.copy(), plan_groups=1)
    g, _ = gpu_encode(x, 512, send.copy())
    assert g.tobytes() == s.tobytes(), "stream depends on the plan shape"


def test_plan_most_groups():
    """4,097 chunks: the default shape caps at 256 groups, giving 242 groups of 17."""
    n = 4097 * C - 5
    say(f"plan most groups n={n}")
    x = varied(n, 24)
    s, _ = check_encode(x)
    check_roundtrip(s, x)


@pytest.mark.parametrize("nchunks,tail", [(1, 60000), (1, 0), (4, 777), (16, 0), (16, 1)])
@pytest.mark.parametrize("B", [0, 64, 512, 32768])
def test_self_planned_write_equals_the_planner(nchunks, tail, B):
    """A tensor of at most 16 chunks is planned inside the write kernel
    (no planner launches); the stream must equal the one the planner's path
    writes for the same input (plan_groups = 1 forces that path), byte for
    byte, and the oracle's."""
    n = nchunks * C - tail
    say(f"self-planned write n={n} B={B}")
    rng = np.random.default_rng(nchunks * 7 + B)
    x = varied(n, 11 + nchunks)
    cache = None
    if B:
        cache = ((x >> 7) & 0xFF).astype(np.uint8)
        cache[rng.random(n) < 0.002] ^= 1
    s_self, c_self = gpu_encode(x, B, cache)
    s_plan, c_plan = gpu_encode(x, B, cache, plan_groups=1)
    assert s_self.tobytes() == s_plan.tobytes()
    if B:
        assert np.array_equal(c_self, c_plan)
    check_encode(x, B, cache)
    check_roundtrip(s_self, x, B, cache.copy() if B else None)
