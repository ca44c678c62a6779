"""Pins of the oracle's packed storage of the fp4 round trip (4-bit e2m1
codes plus one scale byte per block).  The pages keep the round-tripped
values in bf16; the packed form is this library's storage reading, pinned to
(a) hand-worked bytes and (b) the already pinned round trip: unpacking must
give back exactly the round-tripped values."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "fp4_packed_examples.json")


def _bits(x):
    return torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("mode,key,block", [(oracle.E8M0_B32, "e8m0_b32", 32), (oracle.E4M3_B16, "e4m3_b16", 16)])
def test_pack_worked_examples(mode, key, block):
    for case in json.load(open(GOLD))[key]:
        x = np.zeros(case["pad_to"], dtype=np.float32)
        x[: len(case["block"])] = case["block"]
        codes, scales = oracle.pack(_bits(x), mode)
        got = np.stack([codes & 15, codes >> 4], axis=1).reshape(-1)
        want = np.zeros(case["pad_to"], dtype=np.uint8)
        want[: len(case["codes"])] = case["codes"]
        assert np.array_equal(got, want), (case["_why"], got)
        assert scales.tolist() == [case["scale_byte"]], case["_why"]


@pytest.mark.parametrize("mode,block", [(oracle.E8M0_B32, 32), (oracle.E4M3_B16, 16)])
def test_unpack_of_pack_is_the_round_trip(mode, block):
    """Every finite positive bf16 magnitude, both signs, in blocks whose scale
    sweeps the whole range, plus random N(0, sigma) blocks over many sigmas."""
    allpos = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.concatenate([allpos, allpos | 0x8000, [0, 0x8000]]).astype(np.uint16)
    rng = np.random.default_rng(5)
    rng.shuffle(x)
    pad = (-x.size) % block
    x = np.concatenate([x, np.zeros(pad, np.uint16)])
    sig = np.exp(rng.uniform(-20, 20, size=4000 // block + 1)).repeat(block)[: 4000 // block * block]
    r = _bits(rng.standard_normal(sig.size) * sig)
    for arr in (x, r):
        codes, scales = oracle.pack(arr, mode)
        assert np.array_equal(oracle.unpack(codes, scales, arr.size, mode), oracle.quant(arr, mode))


def test_e8m0_scale_byte_closed_form():
    """The E8M0 byte is log2 of the power-of-two scale plus 127, where the
    scale is pow2_ceil(max(amax, 6*2^-126) / 6)."""
    rng = np.random.default_rng(9)
    x = _bits(rng.standard_normal(32 * 500) * np.exp(rng.uniform(-30, 30, 500)).repeat(32))
    _, scales = oracle.pack(x, oracle.E8M0_B32)
    amax = np.abs(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).float().numpy()).reshape(-1, 32).max(1)
    amax = np.maximum(amax.astype(np.float64), 6 * 2.0**-126)
    want = np.ceil(np.log2(np.float32(amax / 6).astype(np.float64))).astype(int) + 127
    assert np.array_equal(scales.astype(int), want)


def test_code_nibbles_hold_grid_indices():
    """Codes decode to e2m1 grid values times the scale: the magnitudes of the
    round trip divided by the scale are exactly the grid entries the low three
    bits name, and bit 3 is the sign bit of the round-tripped value."""
    rng = np.random.default_rng(11)
    x = _bits(rng.standard_normal(32 * 64))
    codes, scales = oracle.pack(x, oracle.E8M0_B32)
    c = np.stack([codes & 15, codes >> 4], axis=1).reshape(-1)
    y = torch.from_numpy(oracle.quant(x, oracle.E8M0_B32).view(np.int16)).view(torch.bfloat16).float().numpy()
    s = np.ldexp(1.0, scales.astype(int) - 127).repeat(32)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    assert np.array_equal(np.abs(y) / s, grid[c & 7])
    assert np.array_equal(np.signbit(y), (c & 8) != 0)
