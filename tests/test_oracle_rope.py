"""Pins of the oracle's latent rotary embedding against what the pages and the
mathematics fix (no GPU).

Pages: "metrale_model_arch/deepseek_v41_ref/compress.rs" -- yarn_freqs_cis
(the table), attention_any (a new latent group is rotated at its group's
position, then fp4 round-tripped with e4m3 scales); "metrale_model_arch/
attn_v41/forward.rs" -- AttnV41::forward (rope on the latent, then fp4_quant,
then the cache copy).  The rotation itself (apply_rotary) is not printed: the
reading is interleaved pairs of the last rope_dim values, binary32 products
and sums, a bf16 result.
"""
import math

import numpy as np
import pytest
import torch

from oracle import oracle

# YaRN parameters of the compressed layers (the pages print no values; these
# are the model family's published rope settings, a reading)
DIM, L0, BASE, FACTOR, BFAST, BSLOW = 64, 4096, 10000.0, 40.0, 32.0, 1.0


def bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def vals(b):
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def test_table_without_correction_is_plain_rope():
    """factor 1 leaves every frequency at base^(-2i/dim): entry (p, i) is the
    cosine and sine of p times that frequency (closed form, binary64 here; the
    table's binary32 frequency and angle allow p * 2 ulp of phase)."""
    t = oracle.yarn_freqs_cis(DIM, 1001, L0, BASE, 1.0, BFAST, BSLOW)
    i = np.arange(DIM // 2)
    theta = BASE ** (-2.0 * i / DIM)
    for p in (0, 1, 2, 7, 100, 1000):
        a = p * theta
        tol = p * theta * 2.5e-7 + 2e-7
        assert np.all(np.abs(t[p, :, 0] - np.cos(a)) <= tol), p
        assert np.all(np.abs(t[p, :, 1] - np.sin(a)) <= tol), p


def _freq_of(t):
    """Per-pair frequency read back from the table's position-1 row."""
    return np.arctan2(t[1, :, 1].astype(np.float64), t[1, :, 0].astype(np.float64))


def test_table_yarn_frequency_classes():
    """YaRN by its definition: a pair that turns at least beta_fast times over
    the original context keeps its frequency, a pair that turns at most
    beta_slow times is slowed by exactly the factor, and the pairs between get
    a frequency strictly between the two that falls with the pair index."""
    t = oracle.yarn_freqs_cis(DIM, 2, L0, BASE, FACTOR, BFAST, BSLOW)
    f = _freq_of(t)
    i = np.arange(DIM // 2)
    theta = BASE ** (-2.0 * i / DIM)
    turns = L0 * theta / (2 * math.pi)
    kept, slowed = turns >= BFAST, turns <= BSLOW
    assert kept.sum() == 11 and slowed.sum() == 9  # pairs 0..10 and 23..31 at these parameters
    assert np.allclose(f[kept], theta[kept], rtol=3e-7, atol=0)
    assert np.allclose(f[slowed], theta[slowed] / FACTOR, rtol=3e-7, atol=0)
    mid = ~kept & ~slowed
    assert np.all(f[mid] < theta[mid]) and np.all(f[mid] > theta[mid] / FACTOR)
    assert np.all(np.diff(f) < 0)


def test_table_basic_identities():
    t = oracle.yarn_freqs_cis(DIM, 5000, L0, BASE, FACTOR, BFAST, BSLOW)
    assert np.all(t[0, :, 0] == 1.0) and np.all(t[0, :, 1] == 0.0)  # angle 0
    r = t[:, :, 0].astype(np.float64) ** 2 + t[:, :, 1].astype(np.float64) ** 2
    assert np.all(np.abs(r - 1) < 4e-7)
    # angle addition: the turn of p1 + p2 is the product of the turns of p1 and p2
    f = _freq_of(t)
    for p1, p2 in ((3, 4), (100, 250), (1000, 2500)):
        z = (t[p1, :, 0] + 1j * t[p1, :, 1]).astype(np.complex128) * (t[p2, :, 0] + 1j * t[p2, :, 1])
        w = t[p1 + p2, :, 0] + 1j * t[p1 + p2, :, 1]
        assert np.all(np.abs(z - w) <= (p1 + p2) * f * 5e-7 + 1e-6), (p1, p2)


def test_rope_quarter_turn_names_the_pairs():
    """A table entry (cos, sin) = (0, 1) turns pair (x0, x1) into (-x1, x0)
    exactly: it shows which values pair up (2i, 2i+1 of the last rope_dim
    values) and the direction; the values before the rope slice are copied."""
    cols, rd = 48, 16
    x = bf16_bits(np.arange(1, cols + 1) * 0.25)
    table = np.zeros((1, rd // 2, 2), np.float32)
    table[0, :, 1] = 1.0
    y = vals(oracle.rope_rows(x.reshape(1, cols), rd, table, [0])[0])
    xv = vals(x)
    assert np.array_equal(y[:cols - rd], xv[:cols - rd])
    assert np.array_equal(y[cols - rd::2], -xv[cols - rd + 1::2])
    assert np.array_equal(y[cols - rd + 1::2], xv[cols - rd::2])
    # the inverse turn goes back
    z = vals(oracle.rope_rows(bf16_bits(y).reshape(1, cols), rd, table, [0], inverse=True)[0])
    assert np.array_equal(z, xv)


def test_rope_is_complex_multiplication():
    """Pair i of the slice times e^(i a) with a the table angle: the binary64
    complex product rounded to bf16 agrees to within one bf16 unit (the
    binary32 intermediate rounds first)."""
    rng = np.random.default_rng(3)
    rows, cols, rd = 64, 512, 64
    t = oracle.yarn_freqs_cis(rd, 70000, L0, BASE, FACTOR, BFAST, BSLOW)
    x = bf16_bits(rng.standard_normal((rows, cols)))
    pos = rng.integers(0, 70000, size=rows)
    y = vals(oracle.rope_rows(x, rd, t, pos))
    xv = vals(x).astype(np.float64)
    z = (xv[:, cols - rd::2] + 1j * xv[:, cols - rd + 1::2]) * (t[pos, :, 0] + 1j * t[pos, :, 1])
    want = np.stack([z.real, z.imag], axis=-1).reshape(rows, rd)
    got = y[:, cols - rd:].astype(np.float64)
    ulp = np.maximum(np.abs(want), 2.0**-126) * 2.0**-7
    assert np.all(np.abs(got - want) <= ulp)
    assert np.mean(got == vals(bf16_bits(want))) > 0.99
    assert np.array_equal(y[:, :cols - rd], vals(x)[:, :cols - rd])


def test_rope_norm_and_inverse():
    rng = np.random.default_rng(4)
    rows, cols, rd = 32, 512, 64
    t = oracle.yarn_freqs_cis(rd, 140000, L0, BASE, FACTOR, BFAST, BSLOW)
    x = bf16_bits(rng.standard_normal((rows, cols)))
    pos = rng.integers(0, 140000, size=rows)
    y = oracle.rope_rows(x, rd, t, pos)
    xv, yv = vals(x).astype(np.float64), vals(y).astype(np.float64)
    n0 = xv[:, cols - rd::2] ** 2 + xv[:, cols - rd + 1::2] ** 2
    n1 = yv[:, cols - rd::2] ** 2 + yv[:, cols - rd + 1::2] ** 2
    assert np.all(np.abs(n1 - n0) <= n0 * 2.0**-6 + 1e-30)
    back = vals(oracle.rope_rows(y, rd, t, pos, inverse=True)).astype(np.float64)
    assert np.all(np.abs(back - xv) <= np.abs(xv) * 2.0**-6 + np.abs(xv).max() * 2.0**-8)
    with pytest.raises(ValueError):
        oracle.rope_rows(x[:1], rd, t, [140000])


def test_rope_at_position_zero_leaves_the_round_trip():
    """Angle 0 turns nothing: rotated-then-quantised rows at position 0 are the
    plain e4m3-scale round trip (values; the sign of a zero may flip)."""
    rng = np.random.default_rng(5)
    t = oracle.yarn_freqs_cis(64, 1, L0, BASE, FACTOR, BFAST, BSLOW)
    x = bf16_bits(rng.standard_normal((8, 512)))
    got = vals(oracle.latent_rope_quant(x, 64, t, np.zeros(8, np.int64)))
    want = vals(oracle.quant(x.reshape(-1), oracle.E4M3_B16).reshape(8, 512))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("ratio", [1, 4, 128])
def test_latent_position_matches_both_page_rules(ratio):
    """Prefill from position 0 rotates group g at g * ratio; a decode step at
    start_pos completing a group rotates it at start_pos + 1 - ratio."""
    for g in range(0, 50):
        assert oracle.latent_position(g, ratio) == g * ratio
    for start_pos in range(ratio - 1, 40 * ratio, ratio):  # (start_pos + 1) % ratio == 0
        j = (start_pos + 1) // ratio - 1
        assert oracle.latent_position(j, ratio) == start_pos + 1 - ratio
