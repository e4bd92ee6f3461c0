"""Host emulation of the bf16 probability encoding the denoising step uses
between its LM head and the next step's self-conditioning contraction
(no GPU; numpy float32 arithmetic in the kernels' order).

The LM head stores, per (row, 64-column tile t), bf16(exp(y - m_t) * f_t)
with f_t = 2^(m_t log2e - r_t), r_t = ceil(m_t log2e): numerators relative
to the power-of-two reference 2^r_t.  The row combine keeps, per row,
R = ceil(M log2e) (M = max_t m_t), the exponents R - r_t (capped at 255) and
g = 2^(R - M log2e) / L (L = sum of exp(y - M)).  The contraction reads each
value with its exponent subtracted from the bf16 exponent field (a
saturating 16-bit subtraction of shift << 7) and the merge multiplies by g.
These tests check that the encoded values reproduce the softmax: within
bf16 rounding wherever a probability is representable, zero only where it is
negligible.
"""
import numpy as np
import pytest

LOG2E = np.float32(1.4426950408889634)
TILE = 64


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    b = x.astype(np.float32).view(np.uint32)
    return ((b + np.uint32(0x7FFF) + ((b >> 16) & np.uint32(1))) >> 16).astype(np.uint32)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def encode_row(y: np.ndarray):
    """y: float32 logits over V (multiple of 64).  Returns (bits, shift, g)."""
    yt = y.reshape(-1, TILE)
    m = yt.max(axis=1)
    mlog = (m * LOG2E).astype(np.float32)
    r = np.ceil(mlog).astype(np.float32)
    f = np.exp2(mlog - r).astype(np.float32)
    t = (yt - m[:, None]).astype(np.float32)
    e = np.exp2((t * LOG2E).astype(np.float32)).astype(np.float32)
    bits = bf16_bits((e * f[:, None]).astype(np.float32))
    l_t = e.sum(axis=1, dtype=np.float32)  # the tile statistic (relative to m_t)
    M = np.float32(m.max())
    R = np.float32(np.ceil(np.float32(M * LOG2E)))
    L = np.float32((l_t * np.exp2(((m - M) * LOG2E).astype(np.float32))).sum(dtype=np.float32))
    g = np.float32(np.exp2(np.float32(R - np.float32(M * LOG2E))) / L)
    shift = np.clip(R - r, 0, 255).astype(np.uint32)
    return bits, shift, g


def decode_row(bits, shift, g):
    """What the contraction multiplies (exponent subtracted, saturating at 0)
    times the row factor the merge applies."""
    sub = bits.astype(np.int64) - (shift.astype(np.int64)[:, None] << 7)
    scaled = np.maximum(sub, 0).astype(np.uint32)
    return bf16_value(scaled).astype(np.float64).reshape(-1) * np.float64(g)


def softmax64(y: np.ndarray) -> np.ndarray:
    z = y.astype(np.float64)
    z = z - z.max()
    p = np.exp(z)
    return p / p.sum()


def check_row(y: np.ndarray):
    bits, shift, g = encode_row(y.astype(np.float32))
    p = softmax64(y)
    q = decode_row(bits, shift, g)
    big = p >= 2.0 ** -100  # far above the bf16 normal range after scaling
    rel = np.abs(q[big] - p[big]) / p[big]
    # bf16 rounding of the numerator plus the float32 exponent arithmetic
    # (at |y log2e| ~ 1300 an ulp of the exponent argument is 2^-13)
    assert rel.max() <= 2.0 ** -8 + 2.0 ** -10, rel.max()
    # anything decoded as zero is negligible
    assert np.all(p[q == 0] < 2.0 ** -110)
    assert np.abs(q - p).sum() <= 4e-3
    return shift


@pytest.mark.parametrize("seed", range(4))
def test_random_rows(seed):
    rng = np.random.default_rng(seed)
    y = (rng.standard_normal(64 * 512) * rng.uniform(0.5, 8.0)).astype(np.float32)
    check_row(y)


def test_peaked_row_caps_the_exponent():
    """One logit hundreds of nats above the rest: the other tiles' exponents
    hit the 255 cap and those tiles decode to zero."""
    rng = np.random.default_rng(7)
    y = rng.standard_normal(64 * 256).astype(np.float32)
    y[1000] = 400.0
    shift = check_row(y)
    assert shift.max() == 255 and shift.min() == 0


def test_flat_row_needs_no_exponent():
    y = np.full(64 * 64, -3.25, dtype=np.float32)
    shift = check_row(y)
    assert shift.max() == 0


def test_negative_and_large_logits():
    """References below zero and far above: the exponent arithmetic is the
    same on either side."""
    rng = np.random.default_rng(3)
    for base in (-500.0, -40.0, 60.0, 900.0):
        y = (base + rng.standard_normal(64 * 128) * 5.0).astype(np.float32)
        check_row(y)
