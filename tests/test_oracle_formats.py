"""Pins of the oracle's number formats (BF16, OCP E4M3FN) and RoPE frequencies.

Each check compares the oracle with something other than itself: the format
specifications (golden tables under tests/golden/), torch's CPU casts (a
library routine) and high-precision decimal arithmetic.
"""
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip() if not line.startswith("#") else ""
            if line:
                rows.append(line.split())
    return rows


# ---------------------------------------------------------------- BF16

def test_bf16_golden_points():
    rows = _golden_rows("bf16_values.txt")
    assert len(rows) >= 10
    bits = np.array([int(r[0], 16) for r in rows], np.uint32)
    want = np.array([int(r[1], 16) for r in rows], np.uint16)
    got = oracle.bf16_from_f32(bits.view(np.float32))
    assert (got == want).all(), list(zip(map(hex, bits), map(hex, got), map(hex, want)))


def _stratified_f32_patterns():
    """Every upper half-word (sign, exponent, top 7 fraction bits) combined
    with lower half-words that exercise each rounding case."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xFFFF],
                    np.uint32)
    rnd = np.random.default_rng(7).integers(0, 1 << 16, size=8).astype(np.uint32)
    lows = np.concatenate([lows, rnd])
    return (hi[:, None] | lows[None, :]).reshape(-1)


def test_bf16_matches_torch_rne_stratified():
    pat = _stratified_f32_patterns()
    x = pat.view(np.float32)
    got = oracle.bf16_from_f32(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(x)
    assert (got[~nan] == ref[~nan]).all()
    # NaN stays NaN (exponent all ones, fraction non-zero) with its sign
    g = got[nan]
    assert ((g & 0x7F80) == 0x7F80).all() and ((g & 0x007F) != 0).all()
    assert ((g >> 15) == (pat[nan] >> 31)).all()


@pytest.mark.slow
def test_bf16_matches_torch_rne_exhaustive():
    for chunk in range(16):
        pat = (np.arange(1 << 28, dtype=np.uint64) + (chunk << 28)).astype(np.uint32)
        x = pat.view(np.float32)
        got = oracle.bf16_from_f32(x)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        ok = (got == ref) | np.isnan(x)
        assert ok.all(), hex(int(pat[~ok][0]))


# ---------------------------------------------------------------- E4M3

def test_e4m3_golden_points():
    rows = _golden_rows("e4m3_ocp.txt")
    assert len(rows) >= 20
    vals = np.array([float(r[0]) for r in rows], np.float32)
    want = np.array([int(r[1], 16) for r in rows], np.uint8)
    got = oracle.e4m3_from_f32(vals)
    assert (got == want).all(), list(zip(vals, map(hex, got), map(hex, want)))


def test_e4m3_decode_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.f64_from_e4m3(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]


def test_e4m3_encode_roundtrips_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.f64_from_e4m3(codes).astype(np.float32)
    assert (oracle.e4m3_from_f32(vals) == codes).all()


def test_e4m3_matches_torch_rne_after_clamp_stratified():
    """torch's cast is round-to-nearest-even; saturation is ours to define,
    so compare on inputs clamped to +-448 first (NaN excluded)."""
    pat = _stratified_f32_patterns()
    x = pat.view(np.float32)
    x = x[~np.isnan(x)]
    clamped = np.clip(x, -448.0, 448.0).astype(np.float32)
    got = oracle.e4m3_from_f32(x)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (got == ref).all()


def test_e4m3_dense_sweep_near_every_code_matches_torch():
    """Values at, between and around every pair of neighbouring codes."""
    pos = oracle.f64_from_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    pts = np.concatenate([pos, mids])
    pts32 = pts.astype(np.float32)
    bits = pts32.view(np.uint32)
    around = np.concatenate([(bits.astype(np.int64) + d).astype(np.uint32).view(np.float32)
                             for d in (-2, -1, 0, 1, 2)])
    around = np.concatenate([around, -around])
    around = around[np.isfinite(around)]
    clamped = np.clip(around, -448.0, 448.0).astype(np.float32)
    got = oracle.e4m3_from_f32(around)
    ref = torch.from_numpy(clamped).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert (got == ref).all()


# ---------------------------------------------------------------- RoPE frequency

@pytest.mark.parametrize("theta,R", [(10000.0, 64), (10000.0, 128), (50000.0, 64),
                                     (1000000.0, 128)])
def test_rope_inv_freq_is_correctly_rounded(theta, R):
    """theta^(-2i/R) to 40 digits, then rounded once to FP32."""
    getcontext().prec = 40
    for i in range(R // 2):
        exact = (Decimal(-2 * i) / Decimal(R) * Decimal(theta).ln()).exp()
        want = np.float32(float(exact))       # double then float: safe at this margin
        # guard: the exact value is not within 1e-30 of a float32 midpoint
        assert oracle.rope_inv_freq(theta, i, R) == want


def test_rope_angle_is_one_fp32_product():
    for pos in (0, 1, 7, 4095, 8191, 32767):
        for invf in (1.0, 0.1, 0.01, 1e-4, 0.8659643):
            f = np.float32(invf)
            assert oracle.rope_angle(pos, float(f)) == np.float32(np.float32(pos) * f)
