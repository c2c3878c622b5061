"""A seeded random sweep over sizes, block sizes, value mixes and cache
states, every encode mode checked against the oracle byte for byte (3-bit
zip3 and ciera with their decodes, single-read zip3 and ciera at a random
window base, the hash sender, rANS zip3 and ciera with their decodes).
Sizes lean on the edges: empty and tiny tensors, sizes next to a chunk
(65,536) or a part (16,384) boundary, a few chunks with a ragged tail."""
import numpy as np
import pytest

from gpu_util import (check_encode, check_encode_e0, check_encode_e0_ciera, check_encode_hashed, check_rans,
                      check_roundtrip, require_gpu, say)
from lossless_bf16_tensor_exp_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = 120


def _size(rng):
    pick = int(rng.integers(0, 4))
    if pick == 0:
        return int(rng.integers(0, 100))
    if pick == 1:
        edge = int(rng.choice([16384, 32768, 49152, 65536, 131072]))
        return max(0, edge + int(rng.integers(-9, 10)))
    if pick == 2:
        return int(rng.integers(100, 70000))
    return int(rng.integers(70000, 300000))


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case):
    require_gpu()
    rng = np.random.default_rng(9000 + case)
    n = _size(rng)
    B = int(2 ** rng.integers(6, 17))  # 64 .. 65536
    frac = float(rng.choice([0.0, 0.0005, 0.02, 1.0]))
    x = wl.mixed_small(rng, n)
    cache = wl.perturbed_cache(rng, x, frac) if frac > 0 else ((x >> 7) & 0xFF).astype(np.uint8)
    e0 = int(rng.integers(0, 250))
    say(f"case {case}: n={n} B={B} cache-change={frac} e0={e0}")
    s, _ = check_encode(x)
    check_roundtrip(s, x)
    s, _ = check_encode(x, B, cache.copy())
    check_roundtrip(s, x, B, cache.copy())
    check_encode_e0(x, e0)
    check_encode_e0_ciera(x, B, cache.copy(), e0)
    check_encode_hashed(x, B, cache.copy())
    check_rans(x)
    check_rans(x, B, cache.copy())
