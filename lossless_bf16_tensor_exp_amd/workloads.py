"""Seeded synthetic BF16 tensors shaped like the pages' workloads.

This module only draws random numbers and rounds float32 to BF16; it holds
none of the codec's arithmetic.  The tests and the benchmark feed the same
arrays to the HIP library and to the CPU oracle.

Every generator uses numpy's PCG64 seeded from ``SeedSequence([tag, seed])``
(``tag`` = the workload's number), so a workload is reproducible from its
number and seed alone.  A "flip" is ``bits ^= 0x0080``: the exponent field's
lowest bit toggles, i.e. the value moves by one binade with sign and mantissa
kept.  Shapes follow the pages' settings (CIERA page, section 2: OLMoE-1B-7B
and DeepSeek-MoE-16B shards, W = 4 and 8; exponent change rates of 0.3-0.5 %
per iteration at LR 1e-4; ZipCCL digest, section 3.1: near-Gaussian tensors),
with random-init weights in place of trained ones.
"""
from __future__ import annotations

import numpy as np

CHUNK = 65536


def rng_for(tag: int, seed: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([tag, seed])))


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (round to nearest, ties to even) on the bit
    pattern; returns uint16.  Inputs must be finite."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (b + np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_to_f32(u: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(u, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(rng: np.random.Generator, n: int, std: float) -> np.ndarray:
    return f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(std))


def bernoulli_positions(rng: np.random.Generator, n: int, p: float) -> np.ndarray:
    """Sorted positions of a Bernoulli(p) process over range(n), drawn as
    geometric gaps (exact process, memory proportional to the hits)."""
    if p <= 0.0 or n == 0:
        return np.zeros(0, dtype=np.int64)
    out = []
    pos = -1
    while True:
        k = max(1024, int(n * p * 1.1) + 64)
        gaps = rng.geometric(p, size=k).astype(np.int64)
        cand = pos + np.cumsum(gaps)
        if cand[-1] >= n:
            out.append(cand[cand < n])
            break
        out.append(cand)
        pos = int(cand[-1])
    return np.concatenate(out)


def flip(bits: np.ndarray, positions: np.ndarray) -> None:
    bits[positions] ^= np.uint16(0x0080)


def random_bits(rng: np.random.Generator, n: int) -> np.ndarray:
    """n fair coin flips as a uint16 array of 0/1."""
    raw = np.frombuffer(rng.bytes((n + 7) // 8), dtype=np.uint8)
    return np.unpackbits(raw, count=n).astype(np.uint16)


# --------------------------------------------------------------------------
# Workload 1: one shard, 2^20 values ~ N(0, 0.02); iteration t adds
# N(0, 1e-4) noise to iteration t-1 (float32 add, then BF16 rounding).
# Exponent reuse with B = 256 plus the 3-bit code.
# --------------------------------------------------------------------------
def workload1(n: int = 1 << 20, seed: int = 0):
    rng = rng_for(1, seed)
    x0 = normal_bf16(rng, n, 0.02)
    noise = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-4)
    x1 = f32_to_bf16(bf16_to_f32(x0) + noise)
    return {"name": "shard-1M-N(0,0.02)+N(0,1e-4)", "mode": "ciera", "B": [256], "iters": [x0, x1]}


# --------------------------------------------------------------------------
# Workload 2: gradient-like tensor, 64 Mi values ~ N(0, 1e-3); exactly
# round(0.001 n) positions (drawn without replacement) hold 1e-3 * t(3)
# draws instead.  3-bit code only (zip3), no reuse cache.
# --------------------------------------------------------------------------
def workload2(n: int = 64 << 20, seed: int = 0):
    rng = rng_for(2, seed)
    g = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    k = int(round(0.001 * n))
    if k:
        pos = rng.choice(n, size=k, replace=False) if n <= (1 << 27) else _sample_without_replacement(rng, n, k)
        g[pos] = (rng.standard_t(3, size=k) * 1e-3).astype(np.float32)
    return {"name": "grad-64M-N(0,1e-3)+0.1%t3", "mode": "zip3", "B": [0], "iters": [f32_to_bf16(g)]}


def _sample_without_replacement(rng, n, k):
    picked = np.unique(rng.integers(0, n, size=k + k // 8 + 16))
    while picked.size < k:
        picked = np.unique(np.concatenate([picked, rng.integers(0, n, size=k)]))
    return rng.permutation(picked)[:k]


# --------------------------------------------------------------------------
# Workload 3: OLMoE-like layer, rank-0 share at W = 4.  Tensors (in order):
# 64 experts x {gate, up, down} 2048x1024, attention q/k/v/o 2048x2048,
# router 2048x64, two norms of 2048.  Each flattened tensor is cut into 4
# equal parts and rank 0's parts are concatenated: n = 104,891,392.  All
# values ~ N(0, 0.02).  Update: in the FFN and attention parts, 5 % of the
# 64-value groups are hot and each value of a hot group flips with p = 1/16;
# every FFN/attention value also toggles its lowest mantissa bit with
# p = 1/2.  Router and norms do not change.  One iteration pair; the block
# size is swept over {64, 128, 256, 512, 1024}.
# --------------------------------------------------------------------------
OLMOE_TENSORS = ([("ffn", 2048 * 1024)] * (64 * 3) + [("attn", 2048 * 2048)] * 4
                 + [("router", 2048 * 64)] + [("norm", 2048)] * 2)


def _shard_segments(tensors, world, scale):
    segs = []
    for kind, numel in tensors:
        part = numel // world
        part = max(64, (part // scale) // 64 * 64) if scale > 1 else part
        segs.append((kind, part))
    return segs


def workload3(scale: int = 1, seed: int = 0):
    rng = rng_for(3, seed)
    segs = _shard_segments(OLMOE_TENSORS, 4, scale)
    n = sum(s for _, s in segs)
    x0 = normal_bf16(rng, n, 0.02)
    moving = np.zeros(n, dtype=bool)
    off = 0
    for kind, s in segs:
        if kind in ("ffn", "attn"):
            moving[off:off + s] = True
        off += s
    x1 = x0.copy()
    groups = n // 64
    hot = (rng.random(groups) < 0.05) & moving[::64][:groups]
    hot_vals = np.repeat(hot, 64)
    flips = hot_vals & (rng.random(n, dtype=np.float32) < np.float32(1.0 / 16.0))
    x1[flips] ^= np.uint16(0x0080)
    x1 ^= random_bits(rng, n) & moving.astype(np.uint16)
    return {"name": "olmoe-layer-W4-rank0", "mode": "ciera", "B": [64, 128, 256, 512, 1024],
            "iters": [x0, x1]}


# --------------------------------------------------------------------------
# Workload 4: DeepSeek-MoE-like layer, rank-0 share at W = 8: (64 routed + 2
# shared) experts x 3 matrices 2048x1408, ~ N(0, 0.015); n = 71,368,704.  A
# fixed, seeded 20 % of the B = 128 blocks are hot.  Each of 10 iterations
# flips hot-block values with p = 2.5 % and toggles every value's lowest
# mantissa bit with p = 1/2.  The chain x0 -> x10 runs with persistent caches.
# --------------------------------------------------------------------------
DEEPSEEK_TENSORS = [("ffn", 2048 * 1408)] * (66 * 3)


def workload4(scale: int = 1, seed: int = 0, iterations: int = 10):
    rng = rng_for(4, seed)
    segs = _shard_segments(DEEPSEEK_TENSORS, 8, scale)
    n = sum(s for _, s in segs)
    x = normal_bf16(rng, n, 0.015)
    nblocks = -(-n // 128)
    hot_blocks = rng.random(nblocks) < 0.20
    hot = np.repeat(hot_blocks, 128)[:n]
    hot_idx = np.flatnonzero(hot)
    iters = [x.copy()]
    for _ in range(iterations):
        sel = hot_idx[rng.random(hot_idx.size, dtype=np.float32) < np.float32(0.025)]
        x[sel] ^= np.uint16(0x0080)
        x ^= random_bits(rng, n)
        iters.append(x.copy())
    return {"name": "deepseek-moe-layer-W8-rank0", "mode": "ciera", "B": [128], "iters": iters}


# --------------------------------------------------------------------------
# Workload 5: 10^9-value stress buffer in regions of 2^20 values (last one
# partial).  Region kinds (seeded): 50 % N(0, 0.02), 25 % 0.02 * t(3), 25 %
# one constant from {+0, -0, 1.0, bf16(0.02), 0x0001}.  Then Bernoulli(1e-4)
# positions take a uniform pick of {+0, -0, random subnormal, +Inf, -Inf,
# NaN with random payload 1..127 and random sign}.  x1 = x0 with
# Bernoulli(0.01) flips.  B = 512.
# --------------------------------------------------------------------------
def workload5(n: int = 1_000_000_000, seed: int = 0, region: int = 1 << 20):
    rng = rng_for(5, seed)
    x0 = np.empty(n, dtype=np.uint16)
    nreg = -(-n // region)
    kinds = rng.choice(3, size=nreg, p=[0.5, 0.25, 0.25])  # 0 normal, 1 student-t, 2 constant
    consts = np.array([0x0000, 0x8000, 0x3F80, int(f32_to_bf16(np.array([0.02], np.float32))[0]), 0x0001],
                      dtype=np.uint16)
    const_pick = rng.integers(0, consts.size, size=nreg)
    for r in range(nreg):
        lo, hi = r * region, min(n, (r + 1) * region)
        if kinds[r] == 0:
            x0[lo:hi] = normal_bf16(rng, hi - lo, 0.02)
        elif kinds[r] == 1:
            x0[lo:hi] = f32_to_bf16((rng.standard_t(3, size=hi - lo) * 0.02).astype(np.float32))
        else:
            x0[lo:hi] = consts[const_pick[r]]
    sp = bernoulli_positions(rng, n, 1e-4)
    what = rng.integers(0, 6, size=sp.size)
    sign = (rng.integers(0, 2, size=sp.size).astype(np.uint16) << np.uint16(15))
    payload = rng.integers(1, 128, size=sp.size).astype(np.uint16)
    vals = np.select(
        [what == 0, what == 1, what == 2, what == 3, what == 4, what == 5],
        [np.uint16(0x0000), np.uint16(0x8000), sign | payload, np.uint16(0x7F80), np.uint16(0xFF80),
         sign | np.uint16(0x7F80) | payload]).astype(np.uint16)
    x0[sp] = vals
    x1 = x0.copy()
    # flips move a finite value by one binade; they skip exponents 254 and 255
    # so that no Inf/NaN becomes a huge finite value (which would dominate the
    # variance) and no finite value becomes Inf/NaN
    fp = bernoulli_positions(rng, n, 0.01)
    flip(x1, fp[((x1[fp] >> np.uint16(7)) & np.uint16(0xFF)) < 254])
    return {"name": "stress-1G-mixed-specials", "mode": "ciera", "B": [512], "iters": [x0, x1]}


WORKLOADS = {1: workload1, 2: workload2, 3: workload3, 4: workload4, 5: workload5}


def all_bf16_patterns() -> np.ndarray:
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


SPECIALS = np.array([0x0000, 0x8000, 0x0001, 0x807F, 0x7F80, 0xFF80, 0x7FC1, 0xFF81, 0x7F81, 0xFFFF],
                    dtype=np.uint16)


def mixed_small(rng: np.random.Generator, n: int) -> np.ndarray:
    """Small edge-case tensor: Gaussian at a random scale, Student-t, or raw
    random bit patterns, with a few specials (+-0, subnormals, +-Inf, NaN
    payloads) planted at random positions."""
    kind = int(rng.integers(0, 3))
    if kind == 0:
        x = f32_to_bf16(rng.standard_normal(n, dtype=np.float32) * np.float32(10.0 ** rng.uniform(-6, 2)))
    elif kind == 1:
        x = f32_to_bf16((rng.standard_t(3, n) * 0.01).astype(np.float32))
    else:
        x = rng.integers(0, 65536, size=n, dtype=np.uint32).astype(np.uint16)
    if n:
        sp = rng.choice(n, size=min(n, int(rng.integers(0, 6))), replace=False)
        x[sp] = rng.choice(SPECIALS, size=sp.size)
    return x


def perturbed_cache(rng: np.random.Generator, x: np.ndarray, frac: float) -> np.ndarray:
    """Exponent bytes of x with about frac of them replaced, as a previous
    iteration's cache would differ."""
    cache = ((x >> 7) & 0xFF).astype(np.uint8)
    n = x.size
    if n:
        k = max(1, int(n * frac))
        cache[rng.choice(n, size=min(n, k), replace=False)] ^= np.uint8(rng.integers(1, 256))
    return cache
