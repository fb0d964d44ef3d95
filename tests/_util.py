"""Helpers shared by the GPU parity tests: host<->device moves of the seeded
inputs and the comparison rules.

Comparison rules:
  * slots and V: bit-exact;
  * K stored as BF16: at most 1 BF16 ulp, or |diff| <= 2^-20 * max|row|
    (a rotation can cancel to a value whose BF16 ulp is below FP32 noise;
    the floor is the FP32 store's own bar);
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


BF16_FLOOR = 2.0 ** -20


def bf16_ok(got, ref, row_axes=(-1,), stats=None):
    """Boolean array: element passes the BF16 K bar (see module doc).
    With a dict ``stats``, also counts the elements compared, those more than
    one ulp apart that pass only by the floor, and the exact matches."""
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
        floor = np.abs(gf - rf) <= BF16_FLOOR * rowmax
    ok = np.where(gnan | rnan, gnan & rnan, (ulp <= 1) | floor)
    if stats is not None:
        stats["n"] = stats.get("n", 0) + int(ok.size)
        stats["floor_only"] = stats.get("floor_only", 0) + int(((ulp > 1) & floor & ~(gnan | rnan)).sum())
        stats["exact"] = stats.get("exact", 0) + int((g == r).sum())
    return ok


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


def tq_unpack(pool, bits, H, D, B=16):
    """A TQ pool [num_blocks, block_bytes] -> (codes [num_blocks, B, H, D],
    scale bytes [num_blocks, B, H, D // 16]).  Layout: per block one region
    per kv head; in it B code rows of D * bits / 8 bytes (group q at 2 * bits
    bytes, element i at bits [bits * i, bits * i + bits) of the group's
    little-endian bytes), then D / 16 scale rows of B bytes."""
    pool = np.ascontiguousarray(pool, np.uint8)
    nb = pool.shape[0]
    NG, gb = D // 16, 2 * bits
    cbytes = B * D * bits // 8
    reg = pool.reshape(nb, H, cbytes + B * NG)
    grp = reg[:, :, :cbytes].reshape(nb, H, B, NG, gb).astype(np.uint64)
    word = np.zeros(grp.shape[:-1], np.uint64)
    for k in range(gb):
        word |= grp[..., k] << np.uint64(8 * k)
    shifts = (np.arange(16, dtype=np.uint64) * np.uint64(bits))
    codes = (word[..., None] >> shifts) & np.uint64((1 << bits) - 1)       # [nb, H, B, NG, 16]
    codes = codes.astype(np.uint8).reshape(nb, H, B, D).transpose(0, 2, 1, 3)
    scales = reg[:, :, cbytes:].reshape(nb, H, NG, B).transpose(0, 3, 1, 2)
    return np.ascontiguousarray(codes), np.ascontiguousarray(scales)


# FP32 decisions of the TQ write kernel: its rms, x / rms and ratio of norms
# carry at most ~11 FP32 rounding errors (16-term sum, square roots, one
# division and one product), far inside this relative margin.
TQ_NEAR = 2.0 ** -19
# outside this range of the FP64 sum of squares a group's FP32 sum of
# squares (or its sixteenth) is subnormal, zero or infinite
TQ_SS_LO, TQ_SS_HI = 2.0 ** -121, 2.0 ** 127


def tq_compare(got_codes, got_scales, v_rows, in_dtype, bits, H, D, in_token_stride=None):
    """Tie-aware comparison of a TQ write with the oracle's FP64 encoder.

    got_codes [T, H, D] (sign << (b-1) | magnitude index) and got_scales
    [T, H, D/16] (E4M3 bytes) of tokens 0..T-1 of ``v_rows``.  Codes must be
    equal except where the FP64 |x / rms| lies within TQ_NEAR (relative) of
    a midpoint between magnitudes, and there differ by at most one
    magnitude, with the same sign; scale bytes must be equal except where
    the FP64 ratio of norms lies within TQ_NEAR of an E4M3 rounding
    midpoint, or the group holds a near-tie code that differs, and there
    differ by at most one E4M3 step.  Groups whose sum of squares is outside
    [TQ_SS_LO, TQ_SS_HI] (the FP32 arithmetic of the kernel cannot take
    their decisions) must have the same scale byte (0 below, 448 above:
    the decoded group is then zero, or saturated) and are not compared code
    by code.  Returns counts."""
    import oracle
    u, ss, ratio, codes, scales = oracle.tq_encode_diag(
        v_rows, in_dtype, bits, num_kv_heads=H, head_dim_v=D, in_token_stride=in_token_stride)
    mags = oracle.f64_from_e4m3(oracle.tq_codebook(bits))
    thr = (mags[1:] + mags[:-1]) / 2
    M = 1 << (bits - 1)
    gc = np.asarray(got_codes, np.uint8)
    gs = np.asarray(got_scales, np.uint8)
    T, NG = u.shape[0], D // 16
    in_dom = (ss == 0) | ((ss >= TQ_SS_LO) & (ss <= TQ_SS_HI))        # [T, H, NG]
    in_dom_e = np.repeat(in_dom, 16, axis=-1)
    au = np.abs(u)
    near_e = (np.abs(au[..., None] - thr).min(axis=-1) <= TQ_NEAR * au) & in_dom_e
    code_eq = gc == codes
    sign_eq = (gc >> (bits - 1)) == (codes >> (bits - 1))
    idx_d = np.abs((gc & (M - 1)).astype(np.int32) - (codes & (M - 1)).astype(np.int32))
    bad_code = in_dom_e & ~code_eq & ~(near_e & sign_eq & (idx_d <= 1))
    assert not bad_code.any(), (
        f"{int(bad_code.sum())} TQ codes differ away from a tie; first at "
        f"{np.argwhere(bad_code)[:3].tolist()}")
    grp_code_diff = (~code_eq & in_dom_e).reshape(T, H, NG, 16).any(axis=-1)
    e4 = oracle.f64_from_e4m3(np.arange(0x7F, dtype=np.uint8))
    mids = (e4[1:] + e4[:-1]) / 2
    near_s = np.abs(ratio[..., None] - mids).min(axis=-1) <= TQ_NEAR * ratio
    step = np.abs(_ordered(gs, 8) - _ordered(scales, 8))
    scale_ok = np.where(in_dom & (near_s | grp_code_diff), step <= 1, gs == scales)
    assert scale_ok.all(), (
        f"{int((~scale_ok).sum())} TQ scale bytes differ; first at "
        f"{np.argwhere(~scale_ok)[:3].tolist()}")
    return {"codes": int(in_dom_e.sum()), "near_tie_codes": int(near_e.sum()),
            "near_tie_codes_differ": int((near_e & ~code_eq).sum()),
            "scales": int(gs.size), "near_tie_scales": int((near_s & in_dom).sum()),
            "scales_differ": int((gs != scales).sum()),
            "groups_out_of_fp32_range": int((~in_dom).sum())}


def tq_rows_by_slot(pool, slots, bits, H, D, B=16):
    """Codes [n, H, D] and scale bytes [n, H, D/16] of the given slots of a
    TQ pool (numpy [num_blocks, block_bytes])."""
    codes, scales = tq_unpack(pool, bits, H, D, B)
    s = np.asarray(slots, np.int64)
    return codes[s // B, s % B], scales[s // B, s % B]


def tq_written_mask(num_blocks, bits, H, D, slots, B=16):
    """Boolean mask over a TQ pool [num_blocks, block_bytes]: True at the
    code-row and scale bytes of the given slots."""
    cb, NG = D * bits // 8, D // 16
    region = B * cb + B * NG
    mask = np.zeros((num_blocks, H * region), bool)
    for s in np.asarray(slots, np.int64):
        blk, t = int(s) // B, int(s) % B
        for h in range(H):
            base = h * region
            mask[blk, base + t * cb: base + (t + 1) * cb] = True
            mask[blk, base + B * cb + np.arange(NG) * B + t] = True
    return mask
