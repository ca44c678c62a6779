"""Pins of the oracle's fp4 round trips against what the pages and the
mathematics fix (no GPU).

Page: "metrale_model_arch/deepseek_v41_ref/compress.rs" -- E2M1, FP4_MAX,
to_e2m1_rne, fp4_quant_e8m0_inplace, fp4_quant_e4m3_inplace.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fp4_worked_examples.json")
GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def all_bf16_bits():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def bf16_vals(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def f32_bits_of(x):
    return np.asarray([x], dtype=np.float32).view(np.uint32)[0]


def test_e2m1_worked_midpoints():
    gold = json.load(open(GOLD))["e2m1_midpoints"]["cases"]
    for y, want in gold:
        got = oracle.e2m1_rne(y)
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (y, got, want)


def _nearest_even_code(a):
    """Brute force from the definition: the grid magnitudes nearest to a; when
    two are equally near, the one whose index into the grid (its code) is even.
    Magnitudes at or beyond the top of the grid map to it."""
    if a >= GRID[-1]:
        return GRID[-1]
    dist = [abs(g - a) for g in GRID]  # exact: a is a bf16 value below 6
    best = min(dist)
    near = [i for i, d in enumerate(dist) if d == best]
    if len(near) == 1:
        return GRID[near[0]]
    assert len(near) == 2 and near[1] == near[0] + 1
    return GRID[near[0] if near[0] % 2 == 0 else near[1]]


def test_e2m1_exhaustive_bf16():
    """Every finite bf16 input: the oracle lands on the nearest grid magnitude
    (ties to the even code, beyond 6 the top of the grid) and keeps the sign."""
    vals = bf16_vals(all_bf16_bits())
    vals = vals[np.isfinite(vals)]
    L = oracle.lib()
    for y in vals:
        y = float(y)
        got = L.sckvo_e2m1_rne(y)
        want = _nearest_even_code(abs(y))
        assert abs(got) == want, (y, got, want)
        assert math.copysign(1, got) == math.copysign(1, y)


def test_e2m1_invariants():
    L = oracle.lib()
    xs = np.linspace(-7, 7, 20001, dtype=np.float32)
    ys = [L.sckvo_e2m1_rne(float(x)) for x in xs]
    assert all(b >= a for a, b in zip(ys, ys[1:])), "monotone"
    for g in GRID:
        assert L.sckvo_e2m1_rne(g) == g and L.sckvo_e2m1_rne(-g) == -g
        assert L.sckvo_e2m1_rne(L.sckvo_e2m1_rne(g)) == g


def test_bf16_rne_matches_torch():
    """Library routine: torch's float32 -> bfloat16 conversion (round to nearest even)."""
    rng = np.random.default_rng(1)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = u.view(np.float32)
    f = f[np.isfinite(f)]
    edge = np.array([0.0, -0.0, 1.0, 1.00390625, 1.0 + 2**-8, 1.0 + 3 * 2**-8, 3.3895314e38, 1e-40, -1e-45,
                     2**-133, 2**-134, 1.5 * 2**-134], dtype=np.float32)
    f = np.concatenate([f, edge])
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    L = oracle.lib()
    got = np.array([L.sckvo_f32_to_bf16(float(x)) for x in f], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (f[bad[:5]], got[bad[:5]], want[bad[:5]])


def test_pow2_ceil_closed_form():
    """Closed form: for x = fr * 2^e with 0.5 <= fr < 1, the ceiling power of two
    is 2^(e-1) when fr == 0.5 and 2^e otherwise."""
    rng = np.random.default_rng(2)
    xs = list(np.exp(rng.uniform(-87, 87, 5000)).astype(np.float32))
    xs += [2.0**-126, 2.0**-125, 0.5, 1.0, 2.0, 1.0000001, 0.99999994, 2.0**126, 1.5 * 2.0**-126]
    for x in xs:
        x = float(np.float32(x))
        fr, e = math.frexp(x)
        want = math.ldexp(1.0, e - 1) if fr == 0.5 else math.ldexp(1.0, e)
        assert oracle.pow2_ceil(x) == want, x


def test_e4m3_matches_torch_float8():
    """Library routine: torch's float32 -> float8_e4m3fn cast (round to nearest
    even) over every non-negative bf16 value where the cast is finite, which
    includes every amax / 6 a bf16 block can give below the saturation point."""
    b = bf16_vals(all_bf16_bits()[:0x7F80])  # +0 .. largest finite positive bf16
    vals = np.concatenate([b, b / np.float32(6)])  # the values themselves and every amax / 6
    t = torch.from_numpy(vals.copy()).to(torch.float8_e4m3fn).float().numpy()
    L = oracle.lib()
    checked = 0
    for x, tv in zip(vals, t):
        if not np.isfinite(tv):
            continue
        got = L.sckvo_e4m3_to_f32(L.sckvo_f32_to_e4m3(float(x)))
        assert got == tv, (x, got, tv)
        checked += 1
    assert checked > 34000


def test_e4m3_brute_codes_and_saturation():
    """The 126 positive finite codes decode to the OCP E4M3FN values and
    encode back to themselves; past 448 the reading saturates to 448."""
    L = oracle.lib()
    vals = [L.sckvo_e4m3_to_f32(c) for c in range(1, 0x7F)]
    assert vals == sorted(vals) and vals[0] == 2.0**-9 and vals[-1] == 448.0
    assert vals[7] == 2.0**-6 and vals[6] == 7 * 2.0**-9
    for c in range(0, 0x7F):
        assert L.sckvo_f32_to_e4m3(L.sckvo_e4m3_to_f32(c)) == c
    for x in [448.0, 464.0, 470.0, 1e6]:
        assert L.sckvo_e4m3_to_f32(L.sckvo_f32_to_e4m3(x)) == 448.0
    # the tie between 1.0 and 1.125 goes to the even code (1.0)
    assert L.sckvo_e4m3_to_f32(L.sckvo_f32_to_e4m3(1.0625)) == 1.0


def _block_case(case, mode):
    blk = np.zeros(case["pad_to"], dtype=np.float32)
    blk[: len(case["block"])] = np.array(case["block"], dtype=np.float32)
    bits = torch.from_numpy(blk).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = bf16_vals(oracle.quant(bits, mode))
    return out[: len(case["expect"])]


@pytest.mark.parametrize("mode,key", [(oracle.E8M0_B32, "e8m0_b32"), (oracle.E4M3_B16, "e4m3_b16")])
def test_quant_worked_examples(mode, key):
    for case in json.load(open(GOLD))[key]:
        got = _block_case(case, mode)
        want = np.array(case["expect"], dtype=np.float32)
        assert np.array_equal(got, want), (case["_why"], got, want)
        assert np.array_equal(np.signbit(got), np.signbit(want)), case["_why"]


def _grid_codes(y):
    return np.array([GRID.index(abs(v)) for v in y])


@pytest.mark.parametrize("mode,block", [(oracle.E8M0_B32, 32), (oracle.E4M3_B16, 16)])
def test_quant_block_invariants(mode, block):
    """Random N(0, sigma) blocks over many magnitudes: every output is e2m1 * s
    for the block's scale s (computed here by the closed forms: frexp for the
    power of two, torch's float8 cast for e4m3), and its grid point is a
    nearest one to clamp(v / s, -6, 6)."""
    rng = np.random.default_rng(3)
    nb = 400
    sig = np.exp(rng.uniform(-12, 12, size=(nb, 1))).astype(np.float32)
    x = (rng.standard_normal((nb, block)).astype(np.float32) * sig)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    bits = xb.view(torch.int16).numpy().view(np.uint16)
    out = bf16_vals(oracle.quant(bits.reshape(-1), mode)).reshape(nb, block)
    xv = xb.float().numpy()
    for b in range(nb):
        amax = np.float32(np.max(np.abs(xv[b])))
        if mode == oracle.E8M0_B32:
            amax = max(amax, np.float32(6 * 2.0**-126))
            fr, e = math.frexp(float(np.float32(amax / np.float32(6))))
            s = math.ldexp(1.0, e - 1) if fr == 0.5 else math.ldexp(1.0, e)
        else:
            amax = max(amax, np.float32(6 * 2.0**-9))
            s = float(torch.tensor([float(np.float32(amax / np.float32(6)))]).to(torch.float8_e4m3fn).float())
            if not math.isfinite(s):
                s = 448.0  # reading: saturate past the largest e4m3 value (torch gives NaN there)
        y = out[b] / np.float32(s)
        assert np.all(np.isin(np.abs(y), GRID)), (b, y)
        r = np.clip(xv[b] / np.float32(s), -6, 6)
        dist = np.abs(np.abs(y) - np.abs(r))
        best = np.min(np.abs(np.abs(r)[:, None] - np.array(GRID)[None, :]), axis=1)
        assert np.all(dist <= best + 0), b
        assert np.array_equal(np.signbit(out[b]), np.signbit(xv[b]))


def test_quant_division_hazards_e4m3():
    """Pairs (v, s) where v / s correctly rounded lands exactly on an e2m1
    midpoint but v * (1/s) does not: the oracle must follow true division (the
    pages divide).  Found by search over bf16 v and e4m3 scales s."""
    L = oracle.lib()
    s_vals = np.array(sorted({L.sckvo_e4m3_to_f32(c) for c in range(1, 0x7F)}), dtype=np.float32)
    v = bf16_vals(all_bf16_bits()[:0x7F80])
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    found = 0
    for s in s_vals:
        q = v / s
        qr = v * (np.float32(1) / s)
        hit = np.isin(q, mids) & (q != qr)
        for vv in v[hit][:2]:
            # the block holds vv and 6*s (so the scale is exactly s); check vv's output
            blk = np.zeros(16, dtype=np.float32)
            blk[0] = vv
            blk[1] = np.float32(6) * s
            bits = torch.from_numpy(blk).to(torch.bfloat16)
            if bits.float()[1].item() != float(blk[1]) or bits.float()[0].item() != float(vv):
                continue
            sb = float(torch.tensor([float(np.float32(np.float32(6) * s / np.float32(6)))]).to(
                torch.float8_e4m3fn).float())
            if sb != float(s):
                continue
            out = bf16_vals(oracle.quant(bits.view(torch.int16).numpy().view(np.uint16), oracle.E4M3_B16))
            mid = float(vv / s)
            want = oracle.e2m1_rne(mid) * float(s)
            assert out[0] == np.float32(want), (vv, s, out[0], want)
            found += 1
    assert found > 20
