"""Pins of the oracle's dtype conversions (oracle/convert.py) against torch's own
casts and a brute-force nearest-value search, independent of the formulas in
convert.py: every bf16 bit pattern widens to torch's value; narrowing matches
torch's float32 -> bf16 cast on exact float32 inputs (ties to even, exponent
carries, subnormals, overflow) and, for float64 inputs, the nearest bf16 value
found by search, so a truncating, round-half-up or double-rounding narrowing
fails."""
import numpy as np
import torch

from oracle.convert import round_to_bf16, round_to_f32, to_f64


def torch_bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(bits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def torch_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.asarray(x, dtype=np.float32).copy()).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_to_f64_every_bf16_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        got = to_f64(bits)
    want = torch_bf16_to_f64(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))   # -0 stays -0
    # the explicit dtype argument and int16 views give the same values
    with np.errstate(invalid="ignore"):
        assert np.array_equal(to_f64(bits.view(np.int16))[~nan], want[~nan])


def test_to_f64_float_inputs_are_exact():
    x = np.random.default_rng(0).standard_normal(1000).astype(np.float32)
    assert np.array_equal(to_f64(x), x.astype(np.float64))
    assert to_f64(x).dtype == np.float64


def _float32_cases():
    rng = np.random.default_rng(1)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    finite_hi = hi[(hi & 0x7F800000) != 0x7F800000]
    parts = [finite_hi | 0x8000,            # exact halfway: ties to even
             finite_hi | 0x7FFF,            # just below halfway
             finite_hi | 0x8001,            # just above halfway
             finite_hi | 0xFFFF,            # carries into the exponent at mantissa 0x7f
             finite_hi,                     # already bf16
             rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)]
    u = np.concatenate(parts)
    f = u.view(np.float32)
    return f[np.isfinite(f)]


def test_round_to_bf16_matches_torch_on_float32_inputs():
    f = _float32_cases()
    got = round_to_bf16(f.astype(np.float64))
    want = torch_f32_to_bf16_bits(f)
    assert np.array_equal(got, want)


def test_round_to_bf16_halfway_and_boundary_cases():
    one = 1.0
    ulp = 2.0 ** -7                                     # bf16 spacing in [1, 2)
    cases = [
        (one + ulp / 2, 0x3F80),                        # tie, even neighbour below
        (one + 3 * ulp / 2, 0x3F82),                    # tie, even neighbour above
        (2.0 - ulp / 4, 0x4000),                        # rounds up across the exponent boundary
        (2.0 - ulp / 2, 0x4000),                        # tie between 0x3fff (odd) and 2.0 (even)
        (-(one + ulp / 2), 0xBF80),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (3.4e38, 0x7F80),                               # beyond the largest bf16 + half ulp: inf
    ]
    for x, want in cases:
        assert int(round_to_bf16(np.array([x]))[0]) == want, x


def _nearest_bf16_brute_force(x: float) -> int:
    """Nearest bf16 by search over the neighbouring patterns; ties to the even pattern."""
    f = np.float32(x)
    base = int(np.array([f], dtype=np.float32).view(np.uint32)[0]) >> 16
    best = None
    for b in range(max(0, (base & 0x7FFF) - 2), min(0x7F80, (base & 0x7FFF) + 3)):
        pat = (base & 0x8000) | b
        v = float(to_f64(np.array([pat], dtype=np.uint16))[0])
        d = abs(v - x)
        if best is None or d < best[0] or (d == best[0] and pat % 2 == 0):
            best = (d, pat)
    return best[1]


def test_round_to_bf16_single_rounding_of_float64():
    rng = np.random.default_rng(2)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, size=3000))
    # values just above a bf16 halfway point by less than a float32 ulp: rounding to float32
    # first would create a tie and round to even (down); one rounding goes up
    for mant in range(0, 128, 3):
        base = 1.0 + mant / 128.0
        xs.append(base + 2.0 ** -8 + 2.0 ** -40)
        xs.append(-(base + 2.0 ** -8 + 2.0 ** -40) * 2.0 ** -20)
        xs.append(base + 2.0 ** -8 - 2.0 ** -40)
    got = round_to_bf16(np.array(xs))
    for x, g in zip(xs, got):
        assert int(g) == _nearest_bf16_brute_force(x), x


def test_round_to_f32_matches_torch():
    x = np.random.default_rng(3).standard_normal(100000) * 10.0 ** np.random.default_rng(4).integers(-40, 40, 100000)
    want = torch.from_numpy(x).to(torch.float32).numpy()
    assert np.array_equal(round_to_f32(x), want)
