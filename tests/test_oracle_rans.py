"""Pins of the oracle's rANS modes (zip3 + rANS, ciera + rANS): the ANS
coder that the CIERA page uses for changed exponents (section 3.1) done as
our own range ANS.  CPU only."""
import math

import numpy as np
import pytest

import brute_rans
import oracle
from lossless_bf16_tensor_exp_amd import workloads as wl

C = 65536


def test_freqs_worked_example():
    # h = {5: 3, 9: 1}: m = 4, d = 2, M - d = 4094.  f_5 = floor(3 * 4094 / 4)
    # = 3070, f_9 = floor(4094 / 4) = 1023, sum 4093; the 3 left go to the
    # most frequent symbol, 5: f_5 = 3073.
    h = np.zeros(256, dtype=np.uint32)
    h[5], h[9] = 3, 1
    f = oracle.rans_freqs(h)
    assert f[5] == 3073 and f[9] == 1023 and f.sum() == 4096


def test_freqs_properties():
    rng = np.random.default_rng(1)
    for trial in range(300):
        h = np.zeros(256, dtype=np.uint32)
        k = int(rng.integers(1, 257))
        idx = rng.choice(256, size=k, replace=False)
        h[idx] = rng.integers(1, 16384 // k + 1, size=k)
        f = oracle.rans_freqs(h).astype(np.int64)
        assert f.sum() == 4096
        assert ((f > 0) == (h > 0)).all()
        top = int(np.argmax(h))  # lowest index among the largest
        assert f[top] == f.max()
    h = np.zeros(256, dtype=np.uint32)
    h[200] = 7
    f = oracle.rans_freqs(h)
    assert f[200] == 4096 and f.sum() == 4096


def _payloads(stream, nchunks):
    table = stream[128:128 + 8 * (nchunks + 1)].view(np.uint64)
    return [stream[int(table[c]):int(table[c + 1])] for c in range(nchunks)]


def test_single_symbol_part_needs_no_words():
    x = np.full(1000, 0x3C00, dtype=np.uint16)  # one exponent everywhere
    s, st = oracle.encode_rans(x)
    pay = _payloads(s, 1)
    assert [p.size for p in pay] == [384]  # pad128(12 + 2 + 256)
    p = pay[0]
    assert p[0] == p[1] == 0x78
    assert list(p[4:12].view(np.uint16)) == [128, 0, 0, 0]  # words per part: the 64 states of part 0 only
    assert int(p[12:14].view(np.uint16)[0]) == 4096
    states = p[14:14 + 256].view(np.uint16)
    assert (states[0::2] == 0).all() and (states[1::2] == 1).all()  # every state 2^16
    assert np.array_equal(oracle.decode_rans(s, x.size), x)


def test_one_table_per_chunk_one_stream_per_part():
    """Four parts with different exponent mixes share the chunk's table,
    normalised from the chunk's histogram; each part with coded values has
    a stream of its own (ciera: a part whose blocks are all unchanged has
    none)."""
    rng = np.random.default_rng(12)
    x = np.concatenate([np.full(16384, 0x3C00, np.uint16),            # exponent 120 only
                        wl.normal_bf16(rng, 16384, 1.0),
                        np.full(16384, 0x3F80, np.uint16),            # exponent 127 only
                        wl.normal_bf16(rng, 9000, 1e-3)])
    s, _ = oracle.encode_rans(x)
    pay = _payloads(s, 1)[0]
    e = (x >> 7) & 0xFF
    f = oracle.rans_freqs(np.bincount(e, minlength=256).astype(np.uint32))
    lo, hi = int(pay[0]), int(pay[1])
    assert lo == int(np.flatnonzero(f)[0]) and hi == int(np.flatnonzero(f)[-1])
    assert np.array_equal(pay[12:12 + 2 * (hi - lo + 1)].view(np.uint16), f[lo:hi + 1])
    w = pay[4:12].view(np.uint16).astype(int)
    assert (w >= 128).all()
    assert pay.size == -(-(12 + 2 * (hi - lo + 1) + 2 * int(w.sum())) // 128) * 128
    assert np.array_equal(oracle.decode_rans(s, x.size), x)
    # ciera: only part 1's blocks changed
    cache = e.astype(np.uint8).copy()
    prev = cache.copy()
    prev[16384 + 5] ^= 1
    s, st = oracle.encode_rans(x, 512, prev.copy())
    assert st == {"changed_blocks": 1, "coded": 512}
    pay = _payloads(s, 1)[0]
    w = pay[4:12].view(np.uint16).astype(int)
    assert w[0] == 0 and w[1] >= 128 and w[2] == 0 and w[3] == 0
    r = prev.copy()
    assert np.array_equal(oracle.decode_rans(s, x.size, 512, r), x) and np.array_equal(r, cache)


@pytest.mark.parametrize("sigma", [1.0, 0.02, 1e-3])
def test_coded_size_is_the_information_content(sigma):
    """rANS spends, over a part, the symbols' information sum of
    log2(4096 / f_s) bits, up to the final states: 16 bits per emitted word
    plus the growth of each state above its start 2^16."""
    rng = np.random.default_rng(3)
    x = wl.normal_bf16(rng, 16384, sigma)
    s, _ = oracle.encode_rans(x)
    pay = _payloads(s, 1)[0]
    lo, hi = int(pay[0]), int(pay[1])
    f = np.zeros(256)
    f[lo:hi + 1] = pay[12:12 + 2 * (hi - lo + 1)].view(np.uint16)
    w = pay[12 + 2 * (hi - lo + 1):].view(np.uint16)
    nwords = int(pay[4:6].view(np.uint16)[0])
    assert list(pay[6:12].view(np.uint16)) == [0, 0, 0]
    xs = w[0:128:2].astype(np.float64) + w[1:128:2].astype(np.float64) * 65536.0
    spent = 16 * (nwords - 128) + sum(math.log2(v) - 16 for v in xs)
    e = (x >> 7) & 0xFF
    info = float(np.sum(np.log2(4096.0 / f[e])))
    assert abs(spent - info) <= 0.002 * info + 8, (spent, info)
    # and the normalised table costs little over the empirical entropy
    p = np.bincount(e, minlength=256) / e.size
    ent = -float(np.sum(p[p > 0] * np.log2(p[p > 0]))) * e.size
    assert info <= ent * 1.01 + 64


@pytest.mark.parametrize("sigma", [1.0, 0.02, 1e-3])
def test_rans_is_smaller_than_the_3bit_code_on_gaussians(sigma):
    rng = np.random.default_rng(4)
    x = wl.normal_bf16(rng, 4 * C + 333, sigma)
    r, _ = oracle.encode_rans(x)
    t, _ = oracle.encode(x)
    assert r.size < t.size


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_roundtrip_all_patterns(order):
    x = wl.all_bf16_patterns()
    if order == "shuffled":
        x = x[np.random.default_rng(5).permutation(x.size)]
    s, _ = oracle.encode_rans(x)
    assert np.array_equal(oracle.decode_rans(s, x.size), x)


@pytest.mark.parametrize("B", [64, 512, 65536])
def test_roundtrip_ciera_chain(B):
    rng = np.random.default_rng(B)
    x = wl.mixed_small(rng, 3 * C + 1000)
    cs = np.zeros(x.size, dtype=np.uint8)
    cr = np.zeros(x.size, dtype=np.uint8)
    for it in range(4):
        s, st = oracle.encode_rans(x, B, cs)
        y = oracle.decode_rans(s, x.size, B, cr)
        assert np.array_equal(y, x) and np.array_equal(cs, cr)
        x = x.copy()
        wl.flip(x, rng.choice(x.size, size=x.size // 500, replace=False))


@pytest.mark.parametrize("n", [0, 1, 7, 64, 1000, 16384, 16385, C + 5])
def test_matches_independent_encoder(n):
    rng = np.random.default_rng(900 + n)
    x = wl.mixed_small(rng, n)
    s, _ = oracle.encode_rans(x)
    assert s.tobytes() == brute_rans.encode(x).tobytes()
    for B in (64, 1024):
        cache = wl.perturbed_cache(rng, x, 0.02)
        s, _ = oracle.encode_rans(x, B, cache.copy())
        assert s.tobytes() == brute_rans.encode(x, B, cache).tobytes()


def test_decode_rejects_corruption():
    rng = np.random.default_rng(6)
    x = wl.normal_bf16(rng, C, 0.02)
    s, _ = oracle.encode_rans(x)
    a = int(s[128:136].view(np.uint64)[0])
    nw = int(s[a + 4:a + 6].view(np.uint16)[0])
    lo, hi = int(s[a]), int(s[a + 1])
    words = a + 12 + 2 * (hi - lo + 1)

    def bad(mutate):
        t = s.copy()
        mutate(t)
        with pytest.raises(oracle.OracleError):
            oracle.decode_rans(t, x.size)

    bad(lambda t: t.__setitem__(6, 0))                        # mode byte
    bad(lambda t: t.__setitem__(slice(a + 4, a + 6), np.frombuffer(np.uint16(nw + 1).tobytes(), np.uint8)))
    bad(lambda t: t.__setitem__(a + 12, t[a + 12] ^ 1))       # table no longer sums to 4096
    bad(lambda t: t.__setitem__(words + 256 + 20, t[words + 256 + 20] ^ 0x10))  # a renormalisation word
    bad(lambda t: t.__setitem__(words + 3, t[words + 3] ^ 0x80))                # a final state
    bad(lambda t: t.__setitem__(136, t[136] ^ 0x40))          # chunk table entry
    bad(lambda t: t.__setitem__(4, 1))                        # version


def test_decode_reads_only_the_stream_in_a_larger_buffer():
    """in_size is the buffer's size, as for the 3-bit streams: bytes after
    total_bytes are not read; a buffer shorter than total_bytes is rejected."""
    rng = np.random.default_rng(8)
    x = wl.normal_bf16(rng, 2 * C + 999, 0.02)
    for B in (0, 256):
        cache = wl.perturbed_cache(rng, x, 0.05) if B else None
        s, _ = oracle.encode_rans(x, B, cache.copy() if B else None)
        longer = np.concatenate([s, rng.integers(0, 256, 4096, dtype=np.uint8)])
        assert np.array_equal(oracle.decode_rans(longer, x.size, B, cache.copy() if B else None), x)
        with pytest.raises(oracle.OracleError):
            oracle.decode_rans(s[:-128], x.size, B, cache.copy() if B else None)
