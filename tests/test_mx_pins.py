"""Pins of the MXFP8 oracle (CPU only): the E4M3 element format against
torch's float8_e4m3fn (the same OCP format), the block scale rule of the MX
format against closed forms, and the quantisation error bound.  A slip -- a
wrong exponent bias, rounding away from even, a scale one binade off, a
missing clamp at 448 -- fails at least one."""

import math

import numpy as np
import pytest
import torch

import oracle


def test_e4m3_decode_matches_torch_float8_e4m3fn_on_every_code():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64)
    ours = torch.tensor([oracle.e4m3_decode(c) for c in range(256)], dtype=torch.float64)
    assert torch.equal(torch.isnan(ours), torch.isnan(ref))
    ok = ~torch.isnan(ref)
    assert torch.equal(ours[ok], ref[ok])
    assert oracle.e4m3_decode(0x7E) == oracle.E4M3_MAX and oracle.e4m3_decode(0x01) == 2.0 ** -9


def test_e4m3_round_matches_torch_cast_in_range():
    rng = np.random.default_rng(0)
    grid = sorted({oracle.e4m3_decode(c) for c in range(256) if not math.isnan(oracle.e4m3_decode(c))})
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]            # exact ties
    near = [m + d for m in mids for d in (-1e-6 * max(abs(m), 1e-3), 1e-6 * max(abs(m), 1e-3))]
    rnd = list(rng.uniform(-448, 448, 4000)) + list(rng.standard_normal(4000) * 0.01)
    vals = torch.tensor(grid + mids + near + rnd, dtype=torch.float32)  # fp32 values: no double rounding
    ref = vals.to(torch.float8_e4m3fn).to(torch.float64)
    ours = torch.tensor([oracle.e4m3_round(float(v)) for v in vals], dtype=torch.float64)
    assert torch.equal(ours, ref)


def test_e4m3_saturates_beyond_448():
    for v in (448.0, 449.0, 463.9, 464.0, 500.0, 511.9, 1e9):
        assert oracle.e4m3_round(v) == 448.0 and oracle.e4m3_round(-v) == -448.0


def test_mx_block_on_grid_round_trips_exactly():
    rng = np.random.default_rng(1)
    grid = [oracle.e4m3_decode(c) for c in range(0x7F) if oracle.e4m3_decode(c) >= 0]
    for shared in (-20, -3, 0, 5):
        blk = [float(rng.choice(grid)) * (1 if rng.random() < 0.5 else -1) for _ in range(32)]
        blk[3] = 448.0  # block maximum in [256, 512): the scale is exactly 2^shared
        x = torch.tensor(blk, dtype=torch.float64) * 2.0 ** shared
        codes, scales = oracle.mx_quantize(x.reshape(1, 32))
        assert int(scales[0, 0]) == shared + 127
        assert torch.equal(oracle.mx_dequantize(codes, scales).reshape(32), x)


def test_mx_scale_puts_block_max_in_256_512_and_bounds_the_error():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(40, 128, generator=g, dtype=torch.float64) * torch.logspace(-6, 6, 40, dtype=torch.float64)[:, None]
    x = x.to(torch.bfloat16).to(torch.float64)
    codes, scales = oracle.mx_quantize(x)
    assert codes.shape == (40, 128) and scales.shape == (40, 4)
    deq = oracle.mx_dequantize(codes, scales)
    for r in range(40):
        for blk in range(4):
            xb = x[r, 32 * blk:32 * blk + 32]
            s = 2.0 ** (int(scales[r, blk]) - 127)
            amax = float(xb.abs().max())
            assert 256.0 <= amax / s < 512.0
            err = (deq[r, 32 * blk:32 * blk + 32] - xb).abs()
            # within half a step of the element's binade (2^-4 relative), a
            # subnormal quantum, or the clamp at 448 * s
            bound = torch.maximum(xb.abs() * 2.0 ** -4, torch.full_like(xb, s * 2.0 ** -10))
            clipped = xb.abs() > 448.0 * s
            assert bool(((err <= bound) | clipped).all())
            assert bool((deq[r, 32 * blk:32 * blk + 32][clipped].abs() == 448.0 * s).all())


def test_mx_zero_block_and_signs():
    x = torch.zeros(1, 64, dtype=torch.float64)
    x[0, 40] = -3.0
    codes, scales = oracle.mx_quantize(x)
    assert int(scales[0, 0]) == 127 and int(codes[0, :32].max()) == 0
    assert oracle.mx_dequantize(codes, scales)[0, 40] == -3.0
