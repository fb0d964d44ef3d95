"""Helpers shared by the GPU parity tests: host<->device moves of the seeded
inputs and the comparison rules.

Comparison rules (derived in the design doc):
  * slots and V: bit-exact;
  * K stored as BF16: at most 1 BF16 ulp, or |diff| <= 2^-16 * max|row|
    (a rotation can cancel to a value whose BF16 ulp is below FP32 noise);
  * K stored as E4M3: at most 1 E4M3 step; saturated codes exact;
  * K stored as FP32: |diff| <= 2^-20 * max|row|;
  * attention: max over elements of |gpu - ref| / max|ref row| <= 2e-3.
"""
import numpy as np
import torch

DEV = "cuda"
ATTN_TOL = 2e-3


def dev(a, dtype=None):
    """numpy -> device tensor; uint16 arrays become bfloat16, uint8 E4M3."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    if a.dtype == np.uint8 and dtype is None:
        return torch.from_numpy(a).to(DEV).view(torch.float8_e4m3fn)
    t = torch.from_numpy(a).to(DEV)
    return t if dtype is None else t.to(dtype)


def host(t):
    """device tensor -> numpy (bfloat16 as uint16 bits, E4M3 as uint8 codes)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).cpu().numpy()
    return t.cpu().numpy()


def _ordered(bits, width):
    """Sign-magnitude float patterns -> integers in value order."""
    b = bits.astype(np.int64)
    sign = 1 << (width - 1)
    mag = b & (sign - 1)
    return np.where(b & sign, -mag, mag)


def bf16_ok(got, ref, row_axes=(-1,)):
    """Boolean array: element passes the BF16 K bar (see module doc)."""
    g = got.astype(np.uint16)
    r = ref.astype(np.uint16)
    gnan = (g & 0x7F80) == 0x7F80
    gnan &= (g & 0x7F) != 0
    rnan = (r & 0x7F80) == 0x7F80
    rnan &= (r & 0x7F) != 0
    ulp = np.abs(_ordered(g, 16) - _ordered(r, 16))
    gf = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rf = (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    with np.errstate(invalid="ignore"):
        rowmax = np.nanmax(np.abs(rf), axis=row_axes, keepdims=True)
        floor = np.abs(gf - rf) <= 2.0 ** -16 * rowmax
    return np.where(gnan | rnan, gnan & rnan, (ulp <= 1) | floor)


def e4m3_ok(got, ref):
    g = got.astype(np.uint8)
    r = ref.astype(np.uint8)
    gnan = (g & 0x7F) == 0x7F
    rnan = (r & 0x7F) == 0x7F
    sat = (r & 0x7F) == 0x7E
    ulp = np.abs(_ordered(g, 8) - _ordered(r, 8))
    return np.where(gnan | rnan, gnan & rnan, np.where(sat, g == r, ulp <= 1))


def f32_ok(got, ref, row_axes=(-1,)):
    g = got.astype(np.float64)
    r = ref.astype(np.float64)
    rowmax = np.abs(r).max(axis=row_axes, keepdims=True)
    both_nan = np.isnan(g) & np.isnan(r)
    return both_nan | (np.abs(g - r) <= 2.0 ** -20 * rowmax)


def attn_err(got, ref):
    """max over elements of |got - ref| / max |ref| over the element's row."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max(axis=-1, keepdims=True)
    den = np.where(den > 0, den, 1.0)
    return float((np.abs(got - ref) / den).max())


def say(*a):
    print(*a, flush=True)


def tq_scale_mask(bits, H, D, B=16):
    """Boolean mask over one TQ cache block's bytes: True at scale bytes.
    The block is one region per kv head of B code rows (D * bits / 8 bytes
    each) followed by D / 16 scale rows (B bytes each)."""
    codes, scales = B * D * bits // 8, B * D // 16
    region = np.concatenate([np.zeros(codes, bool), np.ones(scales, bool)])
    return np.tile(region, H)
