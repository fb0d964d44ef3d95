"""Pins of the oracle's TurboQuant-style V cache (b-bit Lloyd-Max codes with
one E4M3 scale per 16 elements and a norm correction; pages 1 and 2 name
these ingredients, the details are the readings stated with the oracle's
code).

Pinned by: the Lloyd-Max optimality conditions of the codebook (centroid and
nearest-neighbour conditions, by numerical integration with scipy), its
symmetry, torch's E4M3 cast of the levels; properties of every coded group
(each code is the nearest level of x / rms, the decoded group has the
input's norm within one E4M3 half-step, signs are kept, zero groups decode
to zero, power-of-two scaling only scales); a hand-worked packing example
(tests/golden/tq3_packing_example.txt); and attention over a TQ cache equal
to attention over an FP32 cache holding the decoded rows.
"""
import os

import numpy as np
import pytest
import torch
from scipy import integrate
from scipy.stats import norm

import oracle
import pkv_workloads as W
from _util import tq_compare, tq_scale_mask, tq_unpack

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_is_lloyd_max_for_the_standard_normal(bits):
    lv = oracle.tq_lloyd_max(bits)
    L = 1 << bits
    assert lv.shape == (L,) and np.all(np.diff(lv) > 0)
    assert np.allclose(lv, -lv[::-1], atol=1e-12)                 # symmetric
    t = np.concatenate([[-np.inf], (lv[1:] + lv[:-1]) / 2, [np.inf]])  # nearest-neighbour cells
    for k in range(L):
        m0, _ = integrate.quad(norm.pdf, t[k], t[k + 1])
        m1, _ = integrate.quad(lambda x: x * norm.pdf(x), t[k], t[k + 1])
        assert abs(m1 / m0 - lv[k]) < 1e-9                      # centroid condition


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_codebook_magnitudes_are_the_e4m3_casts(bits):
    lv = oracle.tq_lloyd_max(bits)
    pos = lv[len(lv) // 2:]
    want = torch.tensor(pos, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.tq_codebook(bits)
    assert (got == want).all() and np.all(np.diff(oracle.f64_from_e4m3(got)) > 0)


def _encode(x, bits, in_dt="f32"):
    """Write rows x [T, H, D] into a TQ pool at slots 0..T-1; return the pool
    and the decoded rows read back through single-token attention."""
    T, H, D = x.shape
    nb = (T + 15) // 16
    pool = np.zeros(nb * oracle.tq_block_bytes(bits, 16, H, D), np.uint8)
    oracle.cache_write_v(x, in_dt, np.arange(T, dtype=np.int64), pool, num_kv_heads=H,
                         head_dim_v=D, block_size=16, cache_dtype=f"tq{bits}")
    return pool


def _decoded(pool, bits, T, H, D):
    """Each token's decoded row: attention of one query over a one-token
    sequence returns that token's V row exactly."""
    nb = (T + 15) // 16
    out = np.zeros((T, H, D))
    kp = np.zeros((nb, 16, H, 16), np.float32)
    q = np.zeros((1, H, 16), np.float32)
    for t in range(T):
        bt = np.full((1, 1), t // 16, np.int32)
        # a table whose only block holds token t at offset t % 16: shift the
        # sequence so that its last token is t
        n = t % 16 + 1
        o = oracle.paged_decode(q, "f32", kp, "f32", pool, f"tq{bits}", bt,
                                np.array([n], np.int32), num_q_heads=H, num_kv_heads=H,
                                head_dim_qk=16, head_dim_v=D, block_size=16, scale=1.0,
                                sliding_window=1)
        out[t] = o[0]
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_group_codes_are_nearest_levels_and_norm_is_corrected(bits):
    rng = np.random.default_rng(bits)
    T, H, D = 6, 2, 32
    x = (rng.standard_normal((T, H, D)) * rng.uniform(0.1, 10, (T, H, 1))).astype(np.float32)
    x[2, 1, 16:] = 0.0                                            # one all-zero group
    x[3, 0, 5] = 0.0                                              # a zero element
    pool = _encode(x, bits)
    dec = _decoded(pool, bits, T, H, D)
    mags = oracle.f64_from_e4m3(oracle.tq_codebook(bits))
    levels = np.concatenate([-mags[::-1], mags])
    for t in range(T):
        for h in range(H):
            for q in range(D // 16):
                g = x[t, h, 16 * q:16 * q + 16].astype(np.float64)
                d = dec[t, h, 16 * q:16 * q + 16]
                if not g.any():
                    assert (d == 0).all()
                    continue
                r = np.sqrt((g * g).mean())
                u = g / r
                dist = np.abs(u[:, None] - levels[None, :])
                # the decoded group is scale x (one level per element): divide
                # by the scale and find each element's level
                scale = np.linalg.norm(d) / np.linalg.norm(levels[np.argmin(dist, axis=1)])
                chosen = np.argmin(np.abs(d[:, None] / scale - levels[None, :]), axis=1)
                # each element's level is a nearest level of x / rms (ties allowed)
                assert np.allclose(dist[np.arange(16), chosen], dist.min(axis=1), atol=1e-9)
                assert np.sign(d[g != 0]).tolist() == np.sign(g[g != 0]).tolist()
                assert abs(np.linalg.norm(d) / np.linalg.norm(g) - 1) <= 2.0 ** -4 + 1e-12


def test_power_of_two_scaling_only_scales():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((3, 2, 32)).astype(np.float32)
    a = _encode(x, 3)
    b = _encode(x * np.float32(4.0), 3)
    sm = tq_scale_mask(3, 2, 32)
    assert sm.size == oracle.tq_block_bytes(3, 16, 2, 32)
    assert (a[~sm] == b[~sm]).all()                               # same codes
    # scale rows: [head][group][token]; tokens 0..2 hold the rows
    sa = oracle.f64_from_e4m3(a[sm]).reshape(2, 2, 16)[:, :, :3]
    sb = oracle.f64_from_e4m3(b[sm]).reshape(2, 2, 16)[:, :, :3]
    assert (sa > 0).all() and np.allclose(sb, 4 * sa)


def test_hand_worked_packing_example():
    rows = {}
    for line in open(os.path.join(GOLDEN, "tq3_packing_example.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            rows[k] = v
    codes = [int(c) for c in rows["codes"]]
    want = bytes(int(b, 16) for b in rows["bytes"])
    # a pool of one block, one head, 16 columns; token 0 holds the group
    blk = oracle.tq_block_bytes(3, 16, 1, 16)
    pool = np.zeros(blk, np.uint8)
    pool[:6] = np.frombuffer(want, np.uint8)
    pool[16 * 6] = 0x38                                           # scale 1.0
    dec = _decoded(pool, 3, 1, 1, 16)[0, 0]
    mags = oracle.f64_from_e4m3(oracle.tq_codebook(3))
    exp = [(-1 if c >> 2 else 1) * mags[c & 3] for c in codes]
    assert dec.tolist() == exp
    # encoder: these decoded values as input give the hand-derived codes
    x = np.array(exp, np.float32).reshape(1, 1, 16)
    enc = _encode(x, 3)
    assert bytes(enc[:6]) == bytes(int(b, 16) for b in rows["encoded_bytes"])


def test_attention_over_tq_cache_equals_attention_over_decoded_rows():
    lay = W.layout(3, num_seqs=3, len_hi=120)
    H, D = 8, 128
    kp = W.e4m3_codes(3, W.S_POOLK, (lay.num_blocks, 16, H, D))
    v = W.normal(3, 95, (lay.num_blocks * 16, H, D))
    pool = np.zeros(lay.num_blocks * oracle.tq_block_bytes(3, 16, H, D), np.uint8)
    oracle.cache_write_v(v, "f32", np.arange(lay.num_blocks * 16, dtype=np.int64), pool,
                         num_kv_heads=H, head_dim_v=D, block_size=16, cache_dtype="tq3")
    # decoded rows of every slot, through single-token attention
    rows = np.zeros((lay.num_blocks * 16, H, D), np.float32)
    q0 = np.zeros((1, H, 16), np.float32)
    k0 = np.zeros((lay.num_blocks, 16, H, 16), np.float32)
    for blk in range(lay.num_blocks):
        for t in range(16):
            rows[blk * 16 + t] = oracle.paged_decode(
                q0, "f32", k0, "f32", pool, "tq3", np.array([[blk]], np.int32),
                np.array([t + 1], np.int32), num_q_heads=H, num_kv_heads=H, head_dim_qk=16,
                head_dim_v=D, block_size=16, scale=1.0, sliding_window=1)[0]
    q = W.queries(3, 3)
    a = oracle.paged_decode(q, "bf16", kp, "fp8", pool, "tq3", lay.block_tables, lay.seq_lens,
                            num_q_heads=64, num_kv_heads=H, head_dim_qk=D, head_dim_v=D,
                            block_size=16, scale=D ** -0.5, k_scale=0.5)
    b = oracle.paged_decode(q, "bf16", kp, "fp8", rows.reshape(lay.num_blocks, 16, H, D), "f32",
                            lay.block_tables, lay.seq_lens, num_q_heads=64, num_kv_heads=H,
                            head_dim_qk=D, head_dim_v=D, block_size=16, scale=D ** -0.5,
                            k_scale=0.5)
    assert np.abs(a - b).max() <= 1e-6 * np.abs(b).max()


def test_hand_worked_ties_example():
    rows = {}
    for line in open(os.path.join(GOLDEN, "tq3_ties_example.txt")):
        if line.strip() and not line.startswith("#"):
            k, *v = line.split()
            rows[k] = v
    x = np.array([float(a) for a in rows["x"]], np.float32).reshape(1, 1, 16)
    enc = _encode(x, 3)
    assert bytes(enc[:6]) == bytes(int(b, 16) for b in rows["bytes"])
    assert enc[16 * 6] == int(rows["scale"][0], 16)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_encoder_diagnostics_match_the_written_pool_and_the_unpacker(bits):
    """tq_encode_diag's codes and scales are those the oracle writes, read
    back by the tests' unpacker of the documented layout; its u is x / rms."""
    rng = np.random.default_rng(20 + bits)
    T, H, D = 40, 3, 48
    x = (rng.standard_normal((T, H, D)) * np.exp(rng.uniform(-3, 3, (T, H, 1)))).astype(np.float32)
    x[7, 1, 16:32] = 0.0
    pool = _encode(x, bits).reshape(-1, oracle.tq_block_bytes(bits, 16, H, D))
    codes, scales = tq_unpack(pool, bits, H, D)
    u, ss, ratio, dc, ds = oracle.tq_encode_diag(x, "f32", bits, num_kv_heads=H, head_dim_v=D)
    assert (codes.reshape(-1, H, D)[:T] == dc).all()
    assert (scales.reshape(-1, H, D // 16)[:T] == ds).all()
    g = x.astype(np.float64).reshape(T, H, D // 16, 16)
    assert np.allclose(ss, (g * g).sum(-1), rtol=1e-14, atol=0)
    rms = np.sqrt((g * g).mean(-1, keepdims=True))
    with np.errstate(invalid="ignore", divide="ignore"):
        want_u = np.where(rms > 0, g / rms, 0.0)
    assert np.allclose(u.reshape(g.shape), want_u, rtol=1e-14, atol=0)
    assert ((ratio == 0) == (ss == 0)).all()


@pytest.mark.parametrize("bits", [3, 4])
def test_tie_aware_comparison_accepts_the_oracle_and_rejects_planted_errors(bits):
    rng = np.random.default_rng(30 + bits)
    T, H, D = 64, 2, 64
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    _, _, _, codes, scales = oracle.tq_encode_diag(x, "f32", bits, num_kv_heads=H, head_dim_v=D)
    st = tq_compare(codes, scales, x, "f32", bits, H, D)
    assert st["scales_differ"] == 0 and st["near_tie_codes_differ"] == 0
    u = oracle.tq_encode_diag(x, "f32", bits, num_kv_heads=H, head_dim_v=D)[0]
    # a code moved one magnitude where |u| is far from every midpoint
    mags = oracle.f64_from_e4m3(oracle.tq_codebook(bits))
    thr = (mags[1:] + mags[:-1]) / 2
    far = np.abs(np.abs(u)[..., None] - thr).min(-1) > 0.05
    t, h, d = np.argwhere(far & ((codes & ((1 << (bits - 1)) - 1)) == 1))[0]
    bad = codes.copy()
    bad[t, h, d] -= 1
    with pytest.raises(AssertionError):
        tq_compare(bad, scales, x, "f32", bits, H, D)
    # a sign flipped
    bad = codes.copy()
    bad[t, h, d] ^= 1 << (bits - 1)
    with pytest.raises(AssertionError):
        tq_compare(bad, scales, x, "f32", bits, H, D)
    # a scale byte one step off, away from an E4M3 midpoint
    bad = scales.copy()
    bad[0, 0, 0] += 1
    with pytest.raises(AssertionError):
        tq_compare(codes, bad, x, "f32", bits, H, D)
