"""Host checks of the fp32 identities the device quantisers rely on (CPU only).

The device quantisers compute v = fp32(x * inv) and round v to an int8 code by
one fp32 add of 1.5 * 2^23, taking the low byte of the sum's bit pattern, with
no clamp.  This file checks, in numpy fp32 arithmetic (round to nearest even,
as on the GPU):

- the add-and-take-the-low-byte rounding equals round-half-to-even followed by
  the int8 conversion for every fp32 v with 2^-2 <= |v| < 127.5, and gives 0 for
  every smaller magnitude tested;
- |fp32(x * fp32(127 / amax))| <= 127 + 2^-17 whenever |x| <= amax, so v never
  leaves that range and the clamp of the activation quantiser never acts.

The GPU parity tests compare the device codes with the oracle bit for bit; this
pins the two facts behind the kernel's shorter form on every value they cover."""
import numpy as np

C = np.float32(12582912.0)  # 1.5 * 2^23


def _low_byte_code(v):
    s = (v + C).view(np.uint32)
    return (s & np.uint32(0xFF)).astype(np.uint8).view(np.int8).astype(np.int32)


def test_magic_add_rounds_half_to_even_on_every_float_below_127_5():
    lo = int(np.float32(0.25).view(np.uint32))
    hi = int(np.float32(127.5).view(np.uint32))  # exclusive
    step = 1 << 24
    checked = 0
    for a in range(lo, hi, step):
        u = np.arange(a, min(a + step, hi), dtype=np.uint32)
        for sign in (0, 0x80000000):
            v = (u | np.uint32(sign)).view(np.float32)
            want = np.rint(v).astype(np.int32)
            got = _low_byte_code(v)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"v={v[bad[0]]!r}: {got[bad[0]]} != {want[bad[0]]}"
            checked += v.size
    assert checked == 2 * (hi - lo)


def test_magic_add_gives_zero_below_a_quarter():
    r = np.random.default_rng(7)
    u = r.integers(0, int(np.float32(0.25).view(np.uint32)), size=2_000_000, dtype=np.uint32)
    for sign in (0, 0x80000000):
        v = (u | np.uint32(sign)).view(np.float32)
        assert np.all(_low_byte_code(v) == 0)
    assert _low_byte_code(np.array([0.0, -0.0], dtype=np.float32)).tolist() == [0, 0]


def test_ties_go_to_even():
    v = np.arange(-127, 127, dtype=np.float32) + np.float32(0.5)
    want = np.rint(v).astype(np.int32)
    assert np.all(want % 2 == 0)
    assert np.array_equal(_low_byte_code(v), want)


def test_scaled_product_stays_within_127_plus_2_to_minus_17():
    r = np.random.default_rng(11)
    # amax over many binades, including the 1e-5 floor of the quantiser
    amax = np.exp(r.uniform(np.log(1e-5), np.log(1e6), size=4_000_000)).astype(np.float32)
    amax = np.concatenate([amax, np.float32([1e-5, 1.0, 127.0, 3.0e38])])
    inv = np.float32(127.0) / amax
    worst = np.abs(amax * inv)  # |x| = amax is the largest product for a given inv
    assert worst.dtype == np.float32
    assert float(worst.max()) <= 127.0 + 2.0 ** -17
    assert np.all(np.rint(worst) <= 127)
