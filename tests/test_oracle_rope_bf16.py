"""Pins of the oracle's rotary embedding and its storage rounding.

The pages only name RoPE (wzjinhao.cn news article 56682, section
信标查询怎么用: beacons are given the current decode position, recent
queries keep their own).  The oracle reads it as the rotate-half convention
with inverse frequencies held in binary32 and cos/sin held in binary32; these
pins check that reading against the complex-number form, its group
properties and numpy/torch library routines.
"""
import numpy as np
import pytest
import torch


def freqs32(theta, d):
    """binary32 inverse frequencies theta^(-2i/d), evaluated by numpy in binary64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(theta, -(2.0 * i) / d).astype(np.float32).astype(np.float64)


def rope_complex(x, pos, theta):
    """Rotation as complex multiplication of the pairs (x_i, x_{i+d/2}) by
    exp(i * pos * w_i), with cos/sin rounded to binary32 like the reading."""
    d = x.shape[0]
    h = d // 2
    a = pos * freqs32(theta, d)
    z = (x[:h] + 1j * x[h:]) * (np.cos(a).astype(np.float32) + 1j * np.sin(a).astype(np.float32))
    return np.concatenate([z.real, z.imag])


@pytest.mark.parametrize("theta", [1e4, 1e6])
@pytest.mark.parametrize("d", [2, 64, 128])
def test_position_zero_is_identity(orc, theta, d):
    x = np.random.default_rng(0).normal(size=d)
    assert np.array_equal(orc.rope(x, 0, theta), x)


@pytest.mark.parametrize("pos", [1, 7, 2175, 32767])
def test_matches_complex_multiplication(orc, pos):
    rng = np.random.default_rng(pos)
    x = rng.normal(size=128)
    np.testing.assert_allclose(orc.rope(x, pos, 1e6), rope_complex(x, pos, 1e6), rtol=0, atol=1e-13)


def test_norm_preserved(orc):
    rng = np.random.default_rng(1)
    for pos in (3, 100, 5000, 32000):
        x = rng.normal(size=64)
        y = orc.rope(x, pos, 1e4)
        # cos/sin are binary32, so cos^2 + sin^2 = 1 only to ~1e-7
        assert abs(np.linalg.norm(y) / np.linalg.norm(x) - 1.0) < 3e-7


def test_relative_position_property(orc):
    """<R_p q, R_j k> = <q, R_{j-p} k>: attention depends only on offsets."""
    rng = np.random.default_rng(2)
    q, k = rng.normal(size=128), rng.normal(size=128)
    for p, j in [(10, 50), (2175, 100), (300, 300), (4000, 12)]:
        lhs = orc.rope(q, p, 1e6) @ orc.rope(k, j, 1e6)
        rhs = q @ orc.rope(k, j - p, 1e6)
        # binary32 frequencies make the angle p*w - j*w differ from (j-p)*w by
        # at most rounding of the product, far below this bound
        assert abs(lhs - rhs) < 1e-4 * (np.linalg.norm(q) * np.linalg.norm(k))


def test_frequencies_are_binary32_theta_powers(orc):
    """A unit vector on coordinate i rotated by one position lands at
    (cos w_i, sin w_i) with w_i the binary32 frequency."""
    d = 16
    w = freqs32(1e4, d)
    for i in range(d // 2):
        e = np.zeros(d)
        e[i] = 1.0
        y = orc.rope(e, 1, 1e4)
        assert y[i] == float(np.float32(np.cos(w[i])))
        assert y[i + d // 2] == float(np.float32(np.sin(w[i])))


# ---------------------------------------------------------------------------
# bfloat16 rounding (single round-to-nearest-even from binary64)
# ---------------------------------------------------------------------------

def test_bf16_matches_torch_on_binary32_values(orc):
    """For binary32 inputs torch's float32 -> bfloat16 cast is round to
    nearest even, the same single rounding."""
    rng = np.random.default_rng(3)
    x = np.concatenate([
        rng.normal(size=4000).astype(np.float32),
        (rng.normal(size=500) * 1e-38).astype(np.float32),   # subnormal range
        (rng.normal(size=500) * 1e37).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], dtype=np.float32),
    ])
    mine = orc.bf16_from_double(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_halfway_and_double_rounding_cases(orc):
    cases = {
        1.0 + 2.0 ** -8: 0x3F80,            # exact halfway -> even (1.0)
        1.0 + 3 * 2.0 ** -8: 0x3F82,        # halfway between 1+2^-7 and 1+2^-6 -> even (1+2^-6)
        1.0 + 2.0 ** -8 + 2.0 ** -40: 0x3F81,  # just above halfway; a detour via binary32 would give 0x3F80
        1.0 + 2.0 ** -8 - 2.0 ** -40: 0x3F80,
        -(1.0 + 2.0 ** -8 + 2.0 ** -40): 0xBF81,
        2.0 ** 128 * (1 - 2.0 ** -9): 0x7F80,  # rounds up past the largest finite -> inf
        2.0 ** -133: 0x0001,                # smallest bf16 subnormal
        2.0 ** -135: 0x0000,                # a quarter of it rounds to zero
        float("inf"): 0x7F80,
    }
    for v, bits in cases.items():
        assert int(orc.bf16_from_double(v)) == bits, (v, hex(int(orc.bf16_from_double(v))))
    assert int(orc.bf16_from_double(float("nan"))) & 0x7F80 == 0x7F80
