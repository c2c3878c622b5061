"""GPU parity of the hash sender (ciera_encode_hashed): the sender keeps two
64-bit SplitMix64 hashes per block instead of the exponents (CIERA page,
section 3.1).  Its stream must equal the oracle's exact-cache stream for the
same previous exponents (no collisions occur in these inputs: the oracle's
exact comparison and the hashes agree), and the hash cache afterwards must
hold the oracle's block hashes of the new tensor."""
import numpy as np
import pytest

from gpu_util import (check_encode_hashed, check_roundtrip, exps, gpu_encode, gpu_encode_hashed, oracle_encode,
                      require_gpu, say)
from lossless_bf16_tensor_exp_amd import workloads as wl

import oracle

pytestmark = pytest.mark.gpu

BLOCKS = [64, 128, 256, 512, 1024, 4096, 8192, 16384, 32768, 65536]
SIZES = [1, 9, 65, 1000, 65535, 65536, 65537, 3 * 65536 + 12345]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


@pytest.mark.parametrize("B", BLOCKS)
@pytest.mark.parametrize("n", SIZES)
def test_hash_sender_small(n, B):
    say(f"hash sender n={n} B={B}")
    rng = np.random.default_rng(7000 + n + B)
    x = wl.mixed_small(rng, n)
    prev = wl.perturbed_cache(rng, x, 0.01)
    s, _ = check_encode_hashed(x, B, prev)
    check_roundtrip(s, x, B, prev.copy())


@pytest.mark.parametrize("B", [64, 512, 32768])
def test_hash_sender_first_iteration_from_zero_cache(B):
    """A zeroed hash cache stands for all-zero previous exponents: blocks of
    zeros and subnormals count as unchanged, as with a zeroed exponent cache."""
    rng = np.random.default_rng(B)
    n = 5 * 65536 + 300
    x = wl.mixed_small(rng, n)
    x[: 3 * B] &= 0x807F  # exponent field 0: zeros and subnormals
    x[-B:] &= 0x807F
    g, hc = gpu_encode_hashed(x, B, np.zeros((-(-n // B), 2), dtype=np.uint64))
    o, st = oracle.encode(x, B, np.zeros(n, dtype=np.uint8))
    assert st["changed_blocks"] < -(-n // B)
    assert g.tobytes() == o.tobytes()
    assert np.array_equal(hc, oracle.block_hashes(x, B))


@pytest.mark.parametrize("B", [64, 128, 1024, 65536])
def test_hash_sender_chain_equals_exact_cache_chain(B):
    """Five iterations of sparse exponent flips: each stream from the hash
    sender equals the exact-cache encode's (GPU) and the oracle's."""
    rng = np.random.default_rng(100 + B)
    n = 40 * 65536 - 777
    x = wl.normal_bf16(rng, n, 0.02)
    send = np.zeros(n, dtype=np.uint8)
    hc = np.zeros((-(-n // B), 2), dtype=np.uint64)
    for it in range(5):
        say(f"  chain B={B} iteration {it}")
        g, hc = gpu_encode_hashed(x, B, hc)
        e, send_after = gpu_encode(x, B, send)
        assert g.tobytes() == e.tobytes(), f"iteration {it}: hash and exact senders differ"
        o, _ = oracle.encode(x, B, send.copy())
        assert g.tobytes() == o.tobytes()
        assert np.array_equal(hc, oracle.block_hashes(x, B))
        send = send_after
        x = x.copy()
        hot = rng.choice(n // 64, size=n // 6400, replace=False)
        pos = (hot[:, None] * 64 + rng.integers(0, 64, (hot.size, 4))).reshape(-1)
        wl.flip(x, np.unique(pos[pos < n]))


def test_hash_sender_deepseek_like_layer():
    """Workload 4 (71,368,704 values, B = 128), the whole ten-iteration
    chain from a zeroed hash cache: each stream equals the oracle's
    exact-cache encode of that iteration, and the hash cache after each
    equals the oracle's block hashes of the tensor just sent."""
    d = wl.workload4()
    it = d["iters"]
    B = 128
    say(f"deepseek-like n={it[0].size} iterations={len(it) - 1}")
    hc = np.zeros((-(-it[0].size // B), 2), dtype=np.uint64)
    prev = np.zeros(it[0].size, dtype=np.uint8)
    for t, x in enumerate(it):
        g, hc = gpu_encode_hashed(x, B, hc)
        o, st = oracle_encode(x, B, prev.copy())
        assert g.tobytes() == o.tobytes(), t
        assert np.array_equal(hc, oracle.block_hashes(x, B)), t
        prev = exps(x)
        say(f"  iter {t} changed={st['changed_blocks']}")