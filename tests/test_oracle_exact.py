"""More pins for the CPU oracle: the exact window statistic, the
chunk-parallel drivers, hash 1 of the block hash, and the largest-stream
bounds.  CPU only.

The window rule (ZipCCL research digest, section 3.1) takes sigma from one
standard-deviation pass; the oracle evaluates it exactly (integer sums per
exponent field, a fixed-size integer comparison with K0 4^k).  The pins
below tie it to exact rationals built independently (tests/brute.py), to
correctly rounded sums of the values (math.fsum) at sizes brute force cannot
reach, and to tensors built so that their variance sits exactly on a window
threshold or a hair below it.
"""
import math
from fractions import Fraction

import numpy as np
import pytest

import brute
import brute_rans
import oracle
from lossless_bf16_tensor_exp_amd import workloads as wl

K0 = Fraction(brute.K0)


def _bf16_of(v: Fraction) -> int:
    """BF16 pattern of a power of two or its negative (exact)."""
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    assert Fraction(2) ** e == a and -126 <= e <= 127
    return sign | ((e + 127) << 7)


def _threshold_tensor(k: int, delta: int, s: int) -> np.ndarray:
    """513 values with mean exactly 0 whose sample variance is exactly
    K0 4^k + delta 4^(k - 17 - s) / 256, delta in {-1, 0, 1}: pairs +-2^j
    (the base-4 digits of a target sum of squares) padded with zeros.

    With 512 = n - 1 and pairs +-a, var = 2 sum(a^2) / 512 = sum(a^2) / 256.
    K0 as a double is an odd integer times 2^-42, so 256 K0 4^k is that odd
    integer times 4^(k - 17); scaled by 4^s, its base-4 digits say how many
    pairs of each power of two make up the sum."""
    target = K0 * Fraction(4) ** k * 256 / Fraction(4) ** (k - 17 - s)
    assert target.denominator == 1
    N = int(target) + delta
    vals = []
    j = 0
    while N:
        d = N % 4
        N //= 4
        a = Fraction(2) ** (k - 17 - s + j)
        vals += [_bf16_of(a), _bf16_of(-a)] * d
        j += 1
    assert len(vals) <= 512
    x = np.zeros(513, dtype=np.uint16)
    x[: len(vals)] = vals
    return np.random.default_rng([k + 200, delta + 1]).permutation(x)


@pytest.mark.parametrize("k", [-100, -40, -11, 0, 30, 100])
def test_window_base_on_and_beside_an_exact_threshold(k):
    s = min(40, k - 17 + 126)  # smallest value 2^(k - 17 - s) stays a normal BF16
    t = K0 * Fraction(4) ** k
    on = _threshold_tensor(k, 0, s)
    below = _threshold_tensor(k, -1, s)
    above = _threshold_tensor(k, 1, s)
    for x, want_var, want_e0 in [(on, t, 127 + k), (below, None, 126 + k), (above, None, 127 + k)]:
        ev, nf = brute.exact_variance(x)
        if want_var is not None:
            assert ev == want_var
        assert (ev >= t) == (want_e0 == 127 + k)
        assert brute.e0_from_exact(ev, nf) == want_e0
        assert oracle.variance(x) == (ev, nf)
        assert oracle.choose_e0(x) == want_e0
    # below differs from the threshold by far less than a double's rounding of it
    if s >= 30:
        assert float(brute.exact_variance(below)[0]) == float(t)


def test_window_base_extremes_exactly():
    # the top of the range: +-max gives var above K0 4^122 -> E0 = 249
    x = np.array([0x7F7F, 0xFF7F], dtype=np.uint16)
    ev, nf = brute.exact_variance(x)
    assert ev > K0 * Fraction(4) ** 122 and oracle.choose_e0(x) == 249
    # the bottom: two smallest subnormals of opposite sign, far below K0 4^-127
    x = np.array([0x0001, 0x8001], dtype=np.uint16)
    ev, nf = brute.exact_variance(x)
    assert 0 < ev < K0 * Fraction(4) ** -127 and oracle.choose_e0(x) == 0
    # a single finite value among non-finite ones: no spread
    assert oracle.choose_e0(np.array([0x7F80, 0x3F80, 0xFFC1], dtype=np.uint16)) == 0


@pytest.mark.parametrize("n", [2, 3, 17, 64, 500, 4097, 20000])
def test_window_base_matches_exact_rationals_at_many_sizes(n):
    rng = np.random.default_rng(n)
    for scale in (1e-30, 1e-3, 0.02, 3.0, 1e20):
        x = wl.f32_to_bf16((rng.standard_normal(n) * scale + scale * rng.standard_normal()).astype(np.float32))
        if n > 4:
            x[rng.choice(n, 3, replace=False)] = np.array([0x0001, 0x7F80, 0xFFC3], dtype=np.uint16)
        ev, nf = brute.exact_variance(x)
        assert oracle.variance(x) == (ev, nf)
        assert oracle.choose_e0(x) == brute.e0_from_exact(ev, nf), scale


def _fsum_variance_interval(x):
    """An interval holding the exact variance, from math.fsum of the values
    and of their squares (each sum correctly rounded, so within a relative
    2^-53 of the exact one; a BF16 value and its square are exact doubles)."""
    e = (x >> 7) & 0xFF
    v = (x[e != 255].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    nf = v.size
    s1 = Fraction(math.fsum(v))
    s2 = Fraction(math.fsum(v * v))
    r = Fraction(1, 2 ** 52)
    s1_lo, s1_hi = sorted([s1 * (1 - r), s1 * (1 + r)])
    sq_hi = max(s1_lo * s1_lo, s1_hi * s1_hi)
    sq_lo = 0 if s1_lo <= 0 <= s1_hi else min(s1_lo * s1_lo, s1_hi * s1_hi)
    lo = (nf * s2 * (1 - r) - sq_hi) / (nf * (nf - 1))
    hi = (nf * s2 * (1 + r) - sq_lo) / (nf * (nf - 1))
    return lo, hi, nf


@pytest.mark.parametrize("kind", ["gaussian", "gradient", "stress"])
def test_exact_variance_at_large_n_against_correctly_rounded_sums(kind):
    rng = np.random.default_rng(17)
    n = 1 << 22
    if kind == "gaussian":
        x = wl.normal_bf16(rng, n, 0.02)
    elif kind == "gradient":
        x = wl.normal_bf16(rng, n, 1e-3)
        pos = rng.choice(n, n // 1000, replace=False)
        x[pos] = wl.f32_to_bf16((rng.standard_t(3, pos.size) * 1e-3).astype(np.float32))
    else:
        x = wl.normal_bf16(rng, n, 0.02)
        x[: n // 4] = 0x3F80  # a constant region of 1.0
        sp = rng.choice(n, n // 1000, replace=False)
        x[sp] = rng.choice(np.array([0, 0x8000, 0x0005, 0x7F80, 0xFF80, 0x7FC7], dtype=np.uint16), sp.size)
    var, nf = oracle.variance(x)
    lo, hi, nf2 = _fsum_variance_interval(x)
    assert nf == nf2 and lo <= var <= hi
    # and the window is the one either end of the interval gives (no threshold inside)
    assert brute.e0_from_exact(lo, nf) == brute.e0_from_exact(hi, nf) == oracle.choose_e0(x)


def test_exponent_sums_by_brute_force():
    rng = np.random.default_rng(3)
    x = rng.integers(0, 65536, 5000, dtype=np.uint32).astype(np.uint16)
    a, b, nf = oracle.exponent_sums(x)
    wa, wb = [0] * 256, [0] * 256
    for v in (int(t) for t in x):
        e = (v >> 7) & 0xFF
        if e == 255:
            continue
        m = (128 if e else 0) + (v & 0x7F)
        wa[e] += -m if v & 0x8000 else m
        wb[e] += m * m
    assert nf == int(np.count_nonzero(((x >> 7) & 0xFF) != 255))
    assert [int(v) for v in a] == wa and [int(v) for v in b] == wb


# ---------------------------------------------------------------- chunk-parallel drivers
@pytest.mark.parametrize("n", [0, 1, 8191, 65536, 3 * 65536 + 777, 1 << 20])
def test_parallel_encode_and_decode_equal_sequential(n):
    rng = np.random.default_rng(n + 1)
    x = wl.normal_bf16(rng, n, 0.02)
    if n:
        x[rng.choice(n, max(1, n // 100), replace=False)] = 0x7FC5
    for B in (0, 64, 512, 65536):
        prev = ((x >> 7) & 0xFF).astype(np.uint8)
        if n:
            prev[rng.choice(n, max(1, n // 5000), replace=False)] ^= 1
        c1 = prev.copy() if B else None
        want, st = oracle.encode(x, B, c1)
        for threads in (1, 3, 8, 64):
            c2 = prev.copy() if B else None
            got, st2 = oracle.encode(x, B, c2, threads=threads)
            assert got.tobytes() == want.tobytes() and st2 == st, (B, threads)
            if B:
                assert np.array_equal(c2, c1)
            r1 = prev.copy() if B else None
            r2 = prev.copy() if B else None
            y1 = oracle.decode(want, n, B, r1)
            y2 = oracle.decode(want, n, B, r2, threads=threads)
            assert np.array_equal(y1, x) and np.array_equal(y2, x)
            if B:
                assert np.array_equal(r1, r2)


def test_parallel_decode_rejects_what_sequential_rejects():
    """Corrupt single bytes of the header, table, escape index and payload:
    the parallel decoder rejects exactly the streams the sequential one
    rejects, and decodes the others to the same values."""
    rng = np.random.default_rng(9)
    n = 5 * 65536 + 99
    x = wl.normal_bf16(rng, n, 1.0)
    good, _ = oracle.zip3_encode(x)
    offs = list(range(0, 200)) + list(rng.integers(200, good.size, 60))
    rejected = 0
    for off in offs:
        bad = good.copy()
        bad[off] ^= 0x5A
        outcome = []
        for threads in (0, 4):
            try:
                outcome.append(oracle.decode(bad, n, threads=threads).tobytes())
            except oracle.OracleError as e:
                outcome.append(e.status)
        assert outcome[0] == outcome[1], off
        rejected += outcome[0] == oracle.ERR_FORMAT
    assert rejected > 100


def test_parallel_encode_forced_window_and_errors():
    rng = np.random.default_rng(2)
    x = wl.normal_bf16(rng, 200000, 0.02)
    for e0 in (0, 116, 249):
        a, _ = oracle.zip3_encode(x, e0_override=e0)
        b, _ = oracle.encode(x, 0, None, e0, threads=5)
        assert a.tobytes() == b.tobytes()
    with pytest.raises(oracle.OracleError):
        oracle.encode(x, 100, np.zeros(x.size, np.uint8), threads=4)  # B not a power of two


# ---------------------------------------------------------------- block hash, both hashes by value
def test_splitmix64_generator_form_equals_the_closed_form():
    for seed, gamma in zip(brute.HASH_SEEDS, brute.HASH_GAMMAS):
        for w in (1, 0x0102030405060708, (1 << 64) - 1):
            g = brute.SplitMix64(w + seed, gamma)
            for k in range(40):
                assert g.next() == brute.splitmix64_mix(w + seed + (k + 1) * gamma)


def test_python_splitmix64_reproduces_published_outputs():
    from conftest import read_golden_ints
    g = read_golden_ints("splitmix64_seed1234567.txt")
    gen = brute.SplitMix64(g["seed"])
    assert [gen.next() for _ in range(5)] == [g[f"out{i}"] for i in range(1, 6)]


@pytest.mark.parametrize("B", [64, 128, 512, 4096, 65536])
def test_both_block_hashes_equal_an_independent_implementation(B):
    rng = np.random.default_rng(B)
    for n in (B, 3 * B + 8, 5 * B - 1, B // 2 + 3):
        x = rng.integers(0, 65536, n, dtype=np.uint32).astype(np.uint16)
        if n > 64:
            x[8:24] &= 0x807F  # two all-zero exponent words
        got = oracle.block_hashes(x, B)
        want = brute.block_hashes(x, B)
        assert [(int(a), int(b)) for a, b in got] == want, n


def test_block_hash_one_values_for_lone_words():
    """Hash 1 of a block whose only nonzero word is w at position k is the
    (k+1)-th output of the generator seeded w + s_1 stepping by g_1."""
    rng = np.random.default_rng(77)
    for k in (0, 1, 7):
        w = int(rng.integers(1, 1 << 62))
        e = np.zeros(64, dtype=np.uint16)
        for i in range(8):
            e[8 * k + i] = (w >> (8 * i)) & 0xFF
        x = (e << 7).astype(np.uint16)
        gen = brute.SplitMix64(w + brute.HASH_SEEDS[1], brute.HASH_GAMMAS[1])
        for _ in range(k + 1):
            want = gen.next()
        assert int(oracle.block_hashes(x, 64)[0, 1]) == want


# ---------------------------------------------------------------- largest streams
def _all_counts(n, B):
    nchunks = -(-n // oracle.CHUNK)
    nc = [min(oracle.CHUNK, n - c * oracle.CHUNK) for c in range(nchunks)]
    nb = [-(-v // B) if B else 0 for v in nc]
    return nb, nc


@pytest.mark.parametrize("B", [0, 64, 256, 65536])
def test_max_encoded_size_is_the_closed_form_at_full_counts(B):
    for n in (0, 1, 127, 128, 65535, 65536, 65537, 3 * 65536 + 5000, 1 << 22):
        nb, nc = _all_counts(n, B)
        assert oracle.max_encoded_size(n, B) == brute.closed_form_size(n, B, nb, nc), n


@pytest.mark.parametrize("B", [0, 64, 512, 65536])
def test_max_encoded_size_is_attained(B):
    """Every value escapes (exponents 0 against a window forced to 249) and
    every block differs from the cache: the stream is exactly the bound."""
    rng = np.random.default_rng(B + 1)
    for n in (1, 1000, 65536 + 7, 2 * 65536):
        x = rng.integers(0, 128, n, dtype=np.uint16) | (rng.integers(0, 2, n, dtype=np.uint16) << 15)
        cache = np.ones(n, dtype=np.uint8) if B else None
        stream, st = oracle.encode(x, B, cache, e0_override=249)
        assert st["escapes"] == n
        assert stream.size == oracle.max_encoded_size(n, B)


@pytest.mark.parametrize("B", [0, 64, 1024])
def test_rans_max_encoded_size_bounds_the_worst_inputs(B):
    """Uniform random exponent fields (the largest entropy, every symbol
    present) and a skewed mix with 255 rare symbols (each at the smallest
    frequency, 12 bits) stay within the bound; the independent encoder gives
    the same size."""
    rng = np.random.default_rng(B + 5)
    for n in (1, 64, 16385, 65536 + 300):
        for kind in ("uniform", "skewed"):
            if kind == "uniform":
                e = rng.integers(0, 256, n)
            else:
                e = np.where(rng.random(n) < 0.9, 120, rng.integers(0, 256, n))
            x = ((e.astype(np.uint16) << 7) | rng.integers(0, 128, n, dtype=np.uint16)).astype(np.uint16)
            cache = np.full(n, 255, dtype=np.uint8) if B else None
            s, _ = oracle.encode_rans(x, B, cache)
            assert s.size <= oracle.rans_max_encoded_size(n, B)
            if n <= 16385:
                assert s.tobytes() == brute_rans.encode(x, B, np.full(n, 255, dtype=np.uint8)).tobytes()


def test_rans_words_per_symbol_bound():
    """The bound charges one 16-bit word per coded symbol plus the flushed
    states: a state stays below 2^32, so each step emits at most one word."""
    rng = np.random.default_rng(1)
    for kind in range(3):
        m = 5000
        sym = list(rng.integers(0, 256, m)) if kind == 0 else [0] * (m - 255) + list(range(1, 256))
        if kind == 2:
            sym = list(rng.permutation(sym))
        hist = [0] * 256
        for s in sym:
            hist[s] += 1
        f = brute_rans.norm_freqs(hist)
        cum = [sum(f[:s]) for s in range(256)]
        words = brute_rans.coded_stream([int(s) for s in sym], f, cum)
        assert len(words) <= 2 * brute_rans.LANES + m
