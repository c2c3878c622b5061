"""The rANS encoder's state update without integer division, checked on the
host: the GPU encoder takes x div f from a FP32 product of x and a value
rfd a little below 1 / f (rounded down from (1 - 2^-22) / f), truncated,
plus one conditional increment.  The bound behind it: for any state
x < f 2^20, p = fl(fl(x) rfd) lies in (x / f - 1/2, x / f], so trunc(p) is
the quotient or one less and r0 = x - trunc(p) f lies in [0, 2 f).

IEEE-754 binary32 with round-to-nearest-even (numpy float32, as the GPU's
v_cvt_f32_u32 and v_mul_f32) is emulated for every f in 1..4096, at the
states next to multiples of f (where truncation errors would show) over the
whole quotient range, and at random states.  CPU only."""
import numpy as np

M = 4096


def rfd_of(f: np.ndarray) -> np.ndarray:
    """(1 - 2^-22) / f rounded down to binary32."""
    v = (1.0 - 2.0 ** -22) / f.astype(np.float64)
    r = v.astype(np.float32)
    up = r.astype(np.float64) > v
    r[up] = np.nextafter(r[up], np.float32(0))
    return r


def states_for(f: int, rng) -> np.ndarray:
    top = f << 20  # states are below f 2^20 when the update runs
    k = np.concatenate([np.arange(0, 1024), np.arange((1 << 20) - 1024, 1 << 20),
                        rng.integers(0, 1 << 20, 1024)]).astype(np.int64)
    x = np.concatenate([k * f - 1, k * f, k * f + f - 1, rng.integers(0, top, 1024), [top - 1]])
    return np.unique(x[(x >= 0) & (x < top)])


def test_rfd_bounds():
    f = np.arange(1, M + 1)
    r = rfd_of(f).astype(np.float64)
    # rfd (1 + 2^-24)^2 < 1 / f  and  rfd > (1 - 2^-21) / f
    assert np.all(r * (1 + 2.0 ** -24) ** 2 * f < 1.0)
    assert np.all(r * f > 1.0 - 2.0 ** -21)


def test_one_sided_quotient_all_f():
    rng = np.random.default_rng(7)
    for f in range(1, M + 1):
        x = states_for(f, rng)
        rfd = rfd_of(np.array([f]))[0]
        p = x.astype(np.uint32).astype(np.float32) * rfd  # two binary32 roundings
        assert p.dtype == np.float32
        # p <= x / f exactly, and p > x / f - 1/2 (p f is exact in float64)
        pf = p.astype(np.float64) * f
        assert np.all(pf <= x) and np.all(pf > x - 0.5 * f), f
        q0 = p.astype(np.int64)  # truncation
        r0 = x - q0 * f
        assert np.all((r0 >= 0) & (r0 < 2 * f)), f
        q = q0 + (r0 >= f)
        assert np.array_equal(q, x // f), f


def test_update_formula_matches_definition():
    # x' = (x div f) M + x mod f + c equals (Q << 12) + x + c - Q f, the
    # form the encoder computes, and stays below 2^32
    rng = np.random.default_rng(8)
    for f in (1, 2, 3, 1000, 2047, 2048, 2049, 4095, 4096):
        x = states_for(f, rng)
        for c in (0, M - f, (M - f) // 2):
            q = x // f
            want = q * M + x % f + c
            got = (q << 12) + x + c - q * f
            assert np.array_equal(want, got)
            assert np.all(want < (1 << 32))
