"""Pins of the oracle's slot mapping, fused K write and V copy.

Pins come from a hand-worked example (tests/golden/slots_worked_example.txt),
closed forms of RMSNorm on special rows, RoPE as multiplication by a unit
complex number (numpy complex arithmetic), and invariants the pages state:
MRoPE with equal positions is bit-identical to the scalar path (page 1,
kv_cache.rs, doc of fused_k_norm_rope_cache_write_bf16_mrope), the V write
copies bytes and touches nothing else (page 1, doc of
reshape_and_cache_flash_v_only).
"""
import os

import numpy as np
import pytest

import oracle
import pkv_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- slots

def _read_slot_example():
    B, T, R, E = None, [], [], []
    with open(os.path.join(GOLDEN, "slots_worked_example.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tag, *vals = line.split()
            vals = [int(v) for v in vals]
            if tag == "B":
                B = vals[0]
            elif tag == "T":
                T.append(vals)
            elif tag == "R":
                R.append(vals)
            elif tag == "E":
                E.extend(vals)
    return B, np.array(T, np.int32), np.array(R, np.int32), np.array(E, np.int64)


def test_slots_worked_example():
    B, bt, runs, expect = _read_slot_example()
    counts = runs[:, 1].astype(np.int64)
    cu = np.concatenate([[0], np.cumsum(counts)])
    got = oracle.fill_slots(bt, runs[:, 0], cu, int(cu[-1]), B)
    assert (got == expect).all(), (got, expect)


def test_slots_identity_table_is_position():
    bt = np.arange(64, dtype=np.int32).reshape(1, -1)
    for B in (1, 8, 16, 32):
        n = 64 * B - 5
        got = oracle.fill_slots(bt, [0], [0, n], n, B)
        assert (got == np.arange(n)).all()


def test_slots_batched_equals_single_sequence_calls():
    lay = W.layout(1)
    start, cu, _ = W.positions_all(lay)
    allslots = oracle.fill_slots(lay.block_tables, start, cu, int(cu[-1]), lay.block_size)
    for s in range(lay.num_seqs):
        one = oracle.fill_slots(lay.block_tables[s], [0], [0, lay.seq_lens[s]],
                                int(lay.seq_lens[s]), lay.block_size)
        assert (allslots[cu[s]:cu[s + 1]] == one).all()


def test_slots_properties_on_shuffled_pool():
    lay = W.layout(2, num_seqs=32)
    start, cu, pos = W.positions_all(lay)
    B = lay.block_size
    slots = oracle.fill_slots(lay.block_tables, start, cu, int(cu[-1]), B)
    seq = np.repeat(np.arange(lay.num_seqs), np.diff(cu))
    # the slot's block is the table entry of the position's block, and the
    # offset in the block is the position's offset
    assert (slots // B == lay.block_tables[seq, pos // B]).all()
    assert (slots % B == pos % B).all()
    # disjoint tables -> distinct slots, all inside the pool, never the pad block
    assert np.unique(slots).size == slots.size
    assert slots.min() >= 0 and slots.max() < lay.num_blocks * B
    assert not (slots // B == lay.pad_block).any()


# ---------------------------------------------------------------- fused K

def _kwrite(k_in, in_dtype, cache_dtype, H, D, *, T=None, w=None, pos=None, nope=False,
            R=None, offset=0, theta=10000.0, eps=1e-6, k_scale=1.0, pos_h=None, pos_w=None):
    T = k_in.shape[0] if T is None else T
    B = 16
    nb = (T + B - 1) // B
    cache = np.zeros((nb, B, H, D), oracle.NP_TYPES[cache_dtype])
    slots = np.arange(T, dtype=np.int64)
    p = np.zeros(T, np.int32) if pos is None else np.asarray(pos, np.int32)
    oracle.cache_write_k(k_in, in_dtype, slots, cache, cache_dtype, num_kv_heads=H,
                         head_dim=D, block_size=B, norm_weight=w, eps=eps, pos_t=p,
                         pos_h=pos_h, pos_w=pos_w, theta=theta, rope_offset=offset,
                         rotary_dim=D if R is None else R, nope=nope, k_scale=k_scale)
    return cache.reshape(nb * B, H, D)[:T]


def test_rmsnorm_constant_row_closed_form():
    """x_j = c for all j: mean(x^2) = c^2, y_j = c / sqrt(c^2 + eps) * w_j."""
    D, eps = 64, 1e-6
    w = np.linspace(0.5, 1.5, D, dtype=np.float32)
    for c in (1.0, -3.0, 0.001, 37.5):
        k = np.full((1, 1, D), c, np.float32)
        y = _kwrite(k, "f32", "f32", 1, D, w=w, nope=True, eps=eps)[0, 0]
        c64 = np.float64(np.float32(c))
        want = c64 / np.sqrt(c64 ** 2 + np.float64(np.float32(eps))) * w.astype(np.float64)
        # FP64 evaluation order differs from the closed form: at most 1 FP32 ulp
        assert (np.abs(y - want) <= np.spacing(np.abs(want).astype(np.float32))).all()


def test_rmsnorm_one_hot_row_closed_form():
    """x = c e_j: mean(x^2) = c^2 / D, so y_j = c / sqrt(c^2/D + eps) ~ sqrt(D)
    and every other element is 0 (fails if the mean used R, or D-1, ...)."""
    D = 128
    w = np.ones(D, np.float32)
    k = np.zeros((1, 1, D), np.float32)
    k[0, 0, 5] = 2.0
    y = _kwrite(k, "f32", "f32", 1, D, w=w, nope=True, eps=0.0)[0, 0]
    assert y[5] == np.float32(np.sqrt(D))
    assert (np.delete(y, 5) == 0).all()


def test_rmsnorm_scale_invariance():
    """Scaling a row by 2^k (exact in BF16) leaves the normalised row unchanged
    when eps is negligible."""
    D, H = 128, 8
    k = W.kv_tokens(2, 16, "k")
    w = W.norm_weight(2)
    base = _kwrite(k, "bf16", "f32", H, D, w=w, nope=True, eps=1e-30)
    for e in (-3, 4):
        ks = oracle.bf16_from_f32(oracle.f32_from_bf16(k) * np.float32(2.0 ** e))
        got = _kwrite(ks, "bf16", "f32", H, D, w=w, nope=True, eps=1e-30)
        assert np.allclose(got, base, rtol=2e-7, atol=0)


def test_rope_pos0_is_identity_and_nope_equals_pos0():
    D, H = 128, 8
    k = W.kv_tokens(2, 8, "k")
    w = W.norm_weight(2)
    normed = _kwrite(k, "bf16", "f32", H, D, w=w, nope=True)
    at0 = _kwrite(k, "bf16", "f32", H, D, w=w, pos=np.zeros(8))
    assert (at0 == normed).all()


def test_rope_is_complex_rotation():
    """NeoX rotate-half RoPE: z_i = y_i + 1j * y_{i+R/2} is multiplied by
    exp(1j * theta_i), theta_i = pos * theta^(-2i/R) (FP32 angle).  Checked with
    numpy's complex exponential on FP32 rows, no norm."""
    D, R, theta = 128, 128, 10000.0
    T = 40
    k = W.normal(2, 77, (T, 1, D))
    pos = np.array([0, 1, 2, 3, 100, 511, 4095, 8191, 16383, 32767] * 4, np.int32)
    got = _kwrite(k, "f32", "f32", 1, D, pos=pos, theta=theta).astype(np.float64)
    i = np.arange(R // 2)
    invf = (np.float64(theta) ** (-2.0 * i / R)).astype(np.float32)
    ang = (pos.astype(np.float32)[:, None] * invf[None, :]).astype(np.float32)
    z = k[:, 0, :R // 2].astype(np.float64) + 1j * k[:, 0, R // 2:R].astype(np.float64)
    zr = z * np.exp(1j * ang.astype(np.float64))
    want = np.concatenate([zr.real, zr.imag], axis=1)
    err = np.abs(got[:, 0, :] - want)
    assert (err <= 4e-7 * np.abs(want).max(axis=1, keepdims=True)).all()


def test_rope_preserves_pair_norms_and_partial_offset():
    """Rotation keeps each pair's norm; with rope_offset=128, R=64 on D=192
    the first 128 dims are untouched (the MLA-style layout)."""
    D, R, off = 192, 64, 128
    T = 12
    k = W.normal(4, 78, (T, 2, D))
    pos = np.arange(T, dtype=np.int32) * 373
    got = _kwrite(k, "f32", "f32", 2, D, pos=pos, R=R, offset=off, theta=50000.0)
    assert (got[..., :off] == k[..., :off]).all()
    a0, b0 = k[..., off:off + R // 2].astype(np.float64), k[..., off + R // 2:].astype(np.float64)
    a1, b1 = got[..., off:off + R // 2].astype(np.float64), got[..., off + R // 2:].astype(np.float64)
    n0, n1 = np.hypot(a0, b0), np.hypot(a1, b1)
    assert np.allclose(n1, n0, rtol=2e-7, atol=1e-30)


def test_relative_position_property():
    """<RoPE_p(q), RoPE_p'(k)> depends only on p - p' (FP64 up to the FP32
    angles; small positions keep the angle rounding below 1e-6)."""
    D = 64
    q = W.normal(0, 80, (1, 1, D))
    k = W.normal(0, 81, (1, 1, D))
    dots = []
    for shift in (0, 3, 10):
        rq = _kwrite(q, "f32", "f32", 1, D, pos=[5 + shift]).astype(np.float64)
        rk = _kwrite(k, "f32", "f32", 1, D, pos=[2 + shift]).astype(np.float64)
        dots.append(float((rq * rk).sum()))
    assert np.allclose(dots, dots[0], rtol=1e-5)


def test_mrope_equal_positions_bit_identical_to_scalar():
    lay = W.layout(1, num_seqs=2)
    _, _, pos = W.positions_all(lay)
    T = pos.size
    k = W.kv_tokens(1, T, "k")
    w = W.norm_weight(1)
    for cdt in ("bf16", "fp8", "f32"):
        a = _kwrite(k, "bf16", cdt, 8, 128, w=w, pos=pos, k_scale=0.05)
        b = _kwrite(k, "bf16", cdt, 8, 128, w=w, pos=pos, pos_h=pos, pos_w=pos, k_scale=0.05)
        assert a.tobytes() == b.tobytes()


def test_mrope_axis_map_is_pair_index_mod_3():
    """With distinct pos_t/pos_h/pos_w, pair i is rotated at the position of
    axis i % 3: the MRoPE row equals, pair by pair, the scalar rows at the
    three positions."""
    D, H, T = 128, 2, 16
    k = W.normal(1, 82, (T, H, D))
    pt = np.arange(T, dtype=np.int32) * 7
    ph = np.arange(T, dtype=np.int32) * 3 + 1000
    pw = np.arange(T, dtype=np.int32) * 11 + 20
    m = _kwrite(k, "f32", "f32", H, D, pos=pt, pos_h=ph, pos_w=pw)
    rows = [_kwrite(k, "f32", "f32", H, D, pos=p) for p in (pt, ph, pw)]
    for i in range(D // 2):
        src = rows[i % 3]
        assert (m[..., i] == src[..., i]).all() and (m[..., i + D // 2] == src[..., i + D // 2]).all()


def test_store_is_single_rounding_of_fp32_value():
    """The BF16 and FP8 stores are the FP32 store rounded once: BF16 is the
    nearest BF16 of the FP32 row (checked with torch's cast), FP8 is within
    half an E4M3 step of row/k_scale and saturates at 448."""
    import torch
    D, H, T = 128, 8, 64
    k = W.kv_tokens(3, T, "k")
    w = W.norm_weight(3)
    pos = np.arange(T, dtype=np.int32) * 500
    f32 = _kwrite(k, "bf16", "f32", H, D, w=w, pos=pos)
    b16 = _kwrite(k, "bf16", "bf16", H, D, w=w, pos=pos)
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (b16 == ref).all()
    ks = float(np.abs(f32).max()) / 448.0 * 0.5          # forces some saturation
    f8 = _kwrite(k, "bf16", "fp8", H, D, w=w, pos=pos, k_scale=ks)
    z = f32.astype(np.float64) / ks
    dec = oracle.f64_from_e4m3(f8)
    sat = np.abs(z) >= 448
    assert sat.any() and (np.abs(dec[sat]) == 448).all()
    # spacing of E4M3 around |z|: 2^(floor(log2|z|) - 3), at least 2^-9
    e = np.floor(np.log2(np.maximum(np.abs(z), 2.0 ** -6)))
    step = 2.0 ** (e - 3)
    assert (np.abs(dec[~sat] - z[~sat]) <= step[~sat] / 2 + 1e-12).all()


def test_k_write_skips_padding_slots_and_keeps_other_rows():
    D, H, T, B = 64, 2, 10, 16
    k = W.kv_tokens(0, T, "k")
    cache = np.full((4, B, H, D), 0x1234, np.uint16)
    slots = np.array([3, -1, 17, 40, -5, 63, 64, 1000, 0, 20], np.int64)
    oracle.cache_write_k(k, "bf16", slots, cache, "bf16", num_kv_heads=H, head_dim=D,
                         block_size=B, norm_weight=W.norm_weight(0), pos_t=np.arange(T))
    rows = cache.reshape(-1, H, D)
    written = {int(s) for s in slots if 0 <= s < 64}
    for r in range(64):
        if r not in written:
            assert (rows[r] == 0x1234).all()
        else:
            assert (rows[r] != 0x1234).any()


# ---------------------------------------------------------------- V copy

def test_v_copy_is_bytewise_and_touches_nothing_else():
    lay = W.layout(1, num_seqs=3)
    start, cu, _ = W.positions_all(lay)
    T = int(cu[-1])
    slots = oracle.fill_slots(lay.block_tables, start, cu, T, lay.block_size)
    slots[::7] = -1                               # padding tokens
    v = W.kv_tokens(1, T, "v")
    pool = np.full((lay.num_blocks, 16, 8, 128), 0xBEEF, np.uint16)
    oracle.cache_write_v(v, "bf16", slots, pool, num_kv_heads=8, head_dim_v=128,
                         block_size=16)
    rows = pool.reshape(-1, 8, 128)
    for t in range(T):
        if slots[t] >= 0:
            assert (rows[slots[t]] == v[t]).all()
    mask = np.ones(rows.shape[0], bool)
    mask[slots[slots >= 0]] = False
    assert (rows[mask] == 0xBEEF).all()


def test_v_copy_fp32_strided_input():
    T, H, D = 9, 4, 64
    stride = H * D + 32
    v = W.normal(4, 83, (T, stride))
    slots = np.array([5, 0, 31, 2, -1, 8, 9, 10, 30], np.int64)
    pool = np.zeros((2, 16, H, D), np.float32)
    oracle.cache_write_v(v, "f32", slots, pool, num_kv_heads=H, head_dim_v=D, block_size=16,
                         in_token_stride=stride)
    rows = pool.reshape(-1, H * D)
    for t in range(T):
        if slots[t] >= 0:
            assert rows[slots[t]].tobytes() == v[t, :H * D].tobytes()
