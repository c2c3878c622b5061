"""Second, independent implementation of the stream layout for tiny inputs.

Pure Python (lists of ints and bit strings), written separately from the C
oracle so that the byte layout -- which the pages leave open -- is pinned by
two implementations agreeing, not by one.  It also computes the variance
with exact rationals, which pins the oracle's FP64 statistic.

Layout (the same reading the oracle implements): header of 128 bytes, chunk
table, escape index (per chunk four u16: escapes before each 16,384-value
quarter), then per 65,536-value chunk the sections sign+mantissa, [bitmap],
three code planes and escapes, each padded to 128 bytes (ZipCCL research
digest, section 3.1; CIERA page, section 3.1).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

CHUNK = 65536
K0 = float.fromhex("0x1.a610ca4a234eep+9")


def exact_value(bits: int) -> Fraction:
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return sign * Fraction(m, 2 ** 133)
    return sign * Fraction(128 + m) * (Fraction(2) ** (e - 134))


def exact_variance(xs) -> tuple[Fraction, int]:
    vals = [exact_value(int(b)) for b in xs if ((int(b) >> 7) & 0xFF) != 255]
    nf = len(vals)
    if nf < 2:
        return Fraction(0), nf
    mean = sum(vals, Fraction(0)) / nf
    return sum(((v - mean) ** 2 for v in vals), Fraction(0)) / (nf - 1), nf


def e0_from_exact(var: Fraction, nf: int) -> int:
    """Window base from the exact variance: integer nearest
    x_opt = log2(sigma) + 0.5 log2(14 ln2 / 16383) (ZipCCL digest, section 3.1),
    evaluated as comparisons with the thresholds K0 * 4^k."""
    if nf < 2 or var <= 0:
        return 0
    best = None
    for k in range(-127, 123):
        if var >= Fraction(K0) * (Fraction(4) ** k):
            best = k
    return 0 if best is None else 127 + best


def _pad(b: bytearray) -> bytearray:
    b.extend(b"\0" * ((-len(b)) % 128))
    return b


def _bits_to_bytes(bits: list[int]) -> bytearray:
    out = bytearray((len(bits) + 7) // 8)
    for t, bit in enumerate(bits):
        if bit:
            out[t // 8] |= 1 << (t % 8)
    return out


def encode(xs, B: int = 0, cache=None, e0: int | None = None) -> bytes:
    """Stream for the list/array of uint16 patterns ``xs``.  ``cache`` (list of
    ints) is read but not modified.  ``e0`` None derives it from the exact
    variance."""
    xs = [int(v) for v in xs]
    n = len(xs)
    if e0 is None:
        e0 = e0_from_exact(*exact_variance(xs))
    exps = [(v >> 7) & 0xFF for v in xs]
    sms = [((v >> 15) << 7) | (v & 0x7F) for v in xs]

    def code(e):
        return e - e0 + 1 if e0 <= e <= e0 + 6 else 0

    nchunks = -(-n // CHUNK)
    table_len = 8 * (nchunks + 1) + 8 * nchunks  # chunk offsets, then the escape index
    base = 128 + table_len + ((-table_len) % 128)
    body = bytearray()
    offsets = []
    index = []  # per chunk: escapes among its values before each quarter
    total_changed = total_esc = 0
    for c in range(nchunks):
        offsets.append(base + len(body))
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        seg = bytearray(bytes(sms[lo:hi]))
        _pad(seg)
        if B:
            blocks = [(j, range(lo + j * B, min(hi, lo + (j + 1) * B))) for j in range(-(-(hi - lo) // B))]
            changed = [any(exps[i] != cache[i] for i in r) for _, r in blocks]
            seg += _pad(_bits_to_bytes([1 if f else 0 for f in changed]))
            slots = []  # (index or None)
            for (j, r), f in zip(blocks, changed):
                if f:
                    idx = list(r)
                    slots += idx + [None] * (B - len(idx))
            total_changed += sum(changed)
        else:
            slots = list(range(lo, hi))
        codes = [code(exps[i]) if i is not None else 0 for i in slots]
        for b in range(3):
            seg += _pad(_bits_to_bytes([(cd >> b) & 1 for cd in codes]))
        esc_at = [i for i, cd in zip(slots, codes) if i is not None and cd == 0]
        esc = bytearray(exps[i] for i in esc_at)
        index.append([sum(1 for i in esc_at if i < lo + q * (CHUNK // 4)) for q in range(4)])
        total_esc += len(esc)
        seg += _pad(esc)
        body += seg
    total = base + len(body)
    offsets.append(total)
    head = bytearray(b"CIER" if B else b"ZIP3")
    head += struct.pack("<HBBQIIQQQQ", 1, 1 if B else 0, e0, n, B, CHUNK, nchunks, total,
                        total_changed, total_esc)
    head += b"\0" * (128 - len(head))
    table = bytearray(struct.pack(f"<{nchunks + 1}Q", *offsets))
    for q4 in index:
        table += struct.pack("<4H", *q4)
    _pad(table)
    return bytes(head + table + body)


def decode_fields(stream: bytes) -> dict:
    """Header fields of a stream (layout reading above)."""
    magic = stream[:4]
    version, mode, e0, n, B, C, nchunks, total, nch, nesc = struct.unpack_from("<HBBQIIQQQQ", stream, 4)
    return {"magic": magic, "version": version, "mode": mode, "E0": e0, "n": n, "B": B, "C": C,
            "nchunks": nchunks, "total_bytes": total, "changed_blocks": nch, "escapes": nesc}


def closed_form_size(n: int, B: int, chunk_changed: list[int], chunk_escapes: list[int]) -> int:
    """Stream size from per-chunk counts: 128 + pad(8 (nc+1) + 8 nc) + sum over
    chunks of pad(n_c) + [ciera] pad(ceil(nb_c/8)) + 3 pad(P_c) + pad(esc_c)."""
    def pad(v):
        return (v + 127) // 128 * 128
    nchunks = -(-n // CHUNK)
    size = 128 + pad(8 * (nchunks + 1) + 8 * nchunks)
    for c in range(nchunks):
        nc = min(CHUNK, n - c * CHUNK)
        size += pad(nc)
        if B:
            size += pad(-(-(-(-nc // B)) // 8))
            plane = chunk_changed[c] * B // 8
        else:
            plane = -(-nc // 8)
        size += 3 * pad(plane) + pad(chunk_escapes[c])
    return size


MASK64 = (1 << 64) - 1
SM64_GAMMA = 0x9E3779B97F4A7C15
# The block hash's two (seed, increment) pairs, as documented with the hash
# sender's entry point: hash 0 is SplitMix64 itself, hash 1 its own pair.
HASH_SEEDS = (0, 0x243F6A8885A308D3)
HASH_GAMMAS = (SM64_GAMMA, 0xD1B54A32D192ED03)


def splitmix64_mix(z: int) -> int:
    """SplitMix64's output function (Steele, Lea and Flood, OOPSLA 2014, with
    the finaliser constants of the published generator)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


class SplitMix64:
    """The generator itself: the state steps by an odd increment, each output
    is the new state through the output function."""

    def __init__(self, seed: int, gamma: int = SM64_GAMMA):
        self.state = seed & MASK64
        self.gamma = gamma

    def next(self) -> int:
        self.state = (self.state + self.gamma) & MASK64
        return splitmix64_mix(self.state)


def block_hashes(xs, B: int) -> list[tuple[int, int]]:
    """The hash sender's two 64-bit hashes of every block of B values (CIERA
    page, section 3.1: a 128-bit block hash from two independent 64-bit
    SplitMix64 hashes).  The block's exponent fields, 8 at a time, form
    little-endian words w_k (the last zero-filled); hash j adds, over the
    nonzero words, the (k+1)-th output of a SplitMix64 generator seeded with
    w_k + s_j and stepping by g_j, i.e. mix(w_k + s_j + (k+1) g_j)."""
    e = [(int(v) >> 7) & 0xFF for v in xs]
    out = []
    for lo in range(0, len(e), B):
        blk = e[lo:lo + B]
        blk += [0] * ((-len(blk)) % 8)
        h = [0, 0]
        for k in range(len(blk) // 8):
            w = sum(blk[8 * k + i] << (8 * i) for i in range(8))
            if w == 0:
                continue
            for j in range(2):
                h[j] = (h[j] + splitmix64_mix(w + HASH_SEEDS[j] + (k + 1) * HASH_GAMMAS[j])) & MASK64
        out.append((h[0], h[1]))
    return out


def window_share(x: float, sigma: float) -> float:
    """P_win(x) = erf(2^(x+7) / (sigma sqrt 2)) - erf(2^x / (sigma sqrt 2))
    (ZipCCL digest, section 3.1)."""
    s = sigma * math.sqrt(2.0)
    return math.erf(2.0 ** (x + 7) / s) - math.erf(2.0 ** x / s)
