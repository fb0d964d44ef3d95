"""Pins of the oracle's FP8 V cache, sliding window and attention sinks.

FP8 V (page 1, kv_cache.rs, reshape_and_cache_fp8: K and V written to FP8
with k_scale and v_scale; decode takes k_scale and v_scale): the store is
checked against the OCP E4M3 reference table (scale 1 and powers of two,
where the division is exact), against the E4M3 error bound and saturation
for other scales, and the decode against decode over an FP32 V pool that
holds the dequantised values.

Sliding window and sinks (pages 1 and 3 pass `sliding_window` and `sinks` to
their decode launchers without stating the semantics; the reading pinned
here: the query at position n-1 sees positions [n - W, n), W = 0 is off; a
sink is one logit per query head that joins the softmax denominator with no
value): checked against numpy/scipy attention over the gathered rows, closed
forms (W = 1 returns the last V row; n = 1 with a sink is a logistic factor),
and invariants (W >= n and a sink of -inf change nothing; table entries
before the window are never read).
"""
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

import oracle
import pkv_workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_golden():
    vals, codes = [], []
    with open(os.path.join(GOLDEN, "e4m3_ocp.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                v, c = line.split()
                vals.append(float(v))
                codes.append(int(c, 16))
    return np.array(vals, np.float32), np.array(codes, np.uint8)


def _vwrite(v, in_dt, slots, H, D, v_scale, nblk=2):
    pool = np.full((nblk, 16, H, D), 0x5A, np.uint8)
    oracle.cache_write_v(v, in_dt, slots, pool, num_kv_heads=H, head_dim_v=D, block_size=16,
                         cache_dtype="fp8", v_scale=v_scale)
    return pool


# ---------------------------------------------------------------- FP8 V store

@pytest.mark.parametrize("v_scale", [1.0, 0.25, 8.0])
def test_fp8_v_store_matches_ocp_table_for_power_of_two_scales(v_scale):
    vals, codes = _e4m3_golden()
    fin = np.isfinite(vals)
    vals, codes = vals[fin], codes[fin]
    n = vals.size
    H, D = 1, 64
    T = (n + D - 1) // D
    v = np.zeros(T * D, np.float32)
    v[:n] = vals * np.float32(v_scale)          # exact: power-of-two scale
    slots = np.arange(T, dtype=np.int64)
    pool = _vwrite(v.reshape(T, D), "f32", slots, H, D, v_scale)
    got = pool.reshape(-1)[:n]
    assert (got == codes).all()


def test_fp8_v_store_error_bound_and_saturation_from_bf16():
    H, D, T = 8, 128, 40
    v = W.kv_tokens(3, T, "v")                  # BF16 bits
    x = oracle.to_f64(v, "bf16")
    vs = float(np.abs(x).max()) / 448.0 * 0.5   # forces some saturation
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    pool = _vwrite(v, "bf16", slots, H, D, vs, nblk=3)
    rows = pool.reshape(-1, H, D)
    dec = oracle.f64_from_e4m3(rows[slots])     # row of token t
    z = x / vs
    sat = np.abs(z) >= 448
    assert sat.any() and (np.abs(dec[sat]) == 448).all()
    assert (np.sign(dec[~sat]) * np.sign(z[~sat]) >= 0).all()
    e = np.floor(np.log2(np.maximum(np.abs(z), 2.0 ** -6)))
    step = 2.0 ** (e - 3)
    assert (np.abs(dec[~sat] - z[~sat]) <= step[~sat] / 2 + 1e-12).all()
    # rows of slots nobody wrote keep their bytes
    untouched = np.ones(rows.shape[0], bool)
    untouched[slots] = False
    assert (rows[untouched] == 0x5A).all()


def test_fp8_v_store_skips_padding_slots_and_same_dtype_is_a_copy():
    H, D, T = 2, 64, 6
    v = W.kv_tokens(0, T, "v")
    slots = np.array([3, -1, 40, 0, 1000, 17], np.int64)
    pool = _vwrite(v, "bf16", slots, H, D, 0.5)
    rows = pool.reshape(-1, H, D)
    for r in range(32):
        if r not in (3, 0, 17):
            assert (rows[r] == 0x5A).all()
    bpool = np.zeros((2, 16, H, D), np.uint16)
    oracle.cache_write_v(v, "bf16", slots, bpool, num_kv_heads=H, head_dim_v=D, block_size=16,
                         cache_dtype="bf16", v_scale=0.5)
    assert (bpool.reshape(-1, H, D)[17] == v[5]).all()


# ---------------------------------------------------------------- FP8 V decode

def _run(q, kp, k_dt, vp, v_dt, lay, Hq, Hkv, scale, **kw):
    return oracle.paged_decode(q, "bf16", kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                               num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=kp.shape[-1],
                               head_dim_v=vp.shape[-1], block_size=16, scale=scale, **kw)


def _rel(got, ref):
    den = np.abs(ref).max(axis=-1, keepdims=True)
    return float((np.abs(got - ref) / np.maximum(den, 1e-300)).max())


def test_fp8_v_decode_equals_decode_over_dequantised_f32_pool():
    lay = W.layout(3, num_seqs=3, len_hi=200)
    kp, vp8 = W.random_pools(3, lay, v_dtype="fp8")
    q = W.queries(3, 3)
    vs = 0.0625 * 3                               # not a power of two
    got = _run(q, kp, "fp8", vp8, "fp8", lay, 64, 8, 128 ** -0.5, k_scale=0.5, v_scale=vs)
    vf = (oracle.f64_from_e4m3(vp8) * vs).astype(np.float32)
    ref = _run(q, kp, "fp8", vf, "f32", lay, 64, 8, 128 ** -0.5, k_scale=0.5)
    assert np.isfinite(got).all()
    assert _rel(got, ref) < 1e-6
    # v_scale is a plain factor on the output
    got2 = _run(q, kp, "fp8", vp8, "fp8", lay, 64, 8, 128 ** -0.5, k_scale=0.5, v_scale=2 * vs)
    assert _rel(got2, 2 * got) < 1e-6


# ---------------------------------------------------------------- window, sinks

def _gather(pool, dt, bt, n, scl=1.0):
    rows = pool.reshape(-1, *pool.shape[2:])
    idx = np.array([bt[t // 16] * 16 + t % 16 for t in range(n)], np.int64)
    x = oracle.to_f64(rows[idx], dt)
    return x * scl if dt == "fp8" else x


def _brute(q, kp, vp, lay, Hq, Hkv, scale, window=0, sinks=None):
    S = len(lay.seq_lens)
    G = Hq // Hkv
    out = np.zeros((S, Hq, vp.shape[-1]))
    qf = oracle.to_f64(q, "bf16")
    for s in range(S):
        n = int(lay.seq_lens[s])
        if n <= 0:
            continue
        lo = n - window if 0 < window < n else 0
        K = _gather(kp, "bf16", lay.block_tables[s], n)[lo:]
        V = _gather(vp, "bf16", lay.block_tables[s], n)[lo:]
        for h in range(Hq):
            sc = scale * (K[:, h // G, :] @ qf[s, h])
            if sinks is not None:
                w = softmax(np.append(sc, sinks[h]))[:-1]   # the sink takes weight, no value
            else:
                w = softmax(sc)
            out[s, h] = w @ V[:, h // G, :]
    return out


@pytest.mark.parametrize("window", [1, 5, 16, 17, 100])
def test_window_matches_brute_force(window):
    lay = W.layout(2, num_seqs=4, len_hi=150)
    lay.seq_lens[:] = [150, 3, 40, 17]
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 4)
    got = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1, sliding_window=window)
    ref = _brute(q, kp, vp, lay, 32, 8, 0.1, window=window)
    assert _rel(got, ref) < 1e-6


def test_window_one_returns_last_v_row_and_wide_window_changes_nothing():
    lay = W.layout(2, num_seqs=3, len_hi=90)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 3)
    got = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1, sliding_window=1)
    rows = vp.reshape(-1, 8, 128)
    for s in range(3):
        n = int(lay.seq_lens[s])
        last = rows[lay.block_tables[s, (n - 1) // 16] * 16 + (n - 1) % 16]
        assert (got[s] == np.repeat(oracle.f32_from_bf16(last), 4, axis=0)).all()
    base = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    wide = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1,
                sliding_window=int(lay.seq_lens.max()))
    assert base.tobytes() == wide.tobytes()


def test_table_entries_before_the_window_are_never_read():
    lay = W.layout(2, num_seqs=2, len_hi=200)
    lay.seq_lens[:] = [200, 130]
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 2)
    a = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1, sliding_window=40)
    bt = lay.block_tables.copy()
    bt[0, :(200 - 40) // 16] = 2 ** 30            # wholly before the window
    bt[1, :(130 - 40) // 16] = -7
    lay2 = W.Layout(lay.index, lay.seq_lens, bt, lay.num_blocks, lay.pad_block, 16)
    b = _run(q, kp, "bf16", vp, "bf16", lay2, 32, 8, 0.1, sliding_window=40)
    assert a.tobytes() == b.tobytes()


def test_sinks_match_brute_force_and_closed_form_factor():
    lay = W.layout(2, num_seqs=3, len_hi=120)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 3)
    sinks = W.normal(2, 77, (32,)) * 3.0
    got = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1, sinks=sinks)
    ref = _brute(q, kp, vp, lay, 32, 8, 0.1, sinks=sinks)
    assert _rel(got, ref) < 1e-6
    # the sink scales the sink-free output by L / (L + e^sink), L = sum e^s
    base = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    qf = oracle.to_f64(q, "bf16")
    for s in range(3):
        n = int(lay.seq_lens[s])
        K = _gather(kp, "bf16", lay.block_tables[s], n)
        for h in range(32):
            lse = logsumexp(0.1 * (K[:, h // 4, :] @ qf[s, h]))
            f = 1.0 / (1.0 + np.exp(float(sinks[h]) - lse))
            assert np.allclose(got[s, h], base[s, h] * f, rtol=1e-6, atol=1e-9)


def test_sink_minus_inf_changes_nothing_and_single_token_is_logistic():
    lay = W.layout(2, num_seqs=2, len_hi=70)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 2)
    base = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    none = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1,
                sinks=np.full(32, -np.inf, np.float32))
    assert base.tobytes() == none.tobytes()
    # n = 1: out = sigma(s0 - sink) v0
    B = 16
    kp1 = np.zeros((1, B, 1, 4), np.float32)
    vp1 = np.zeros((1, B, 1, 3), np.float32)
    kp1[0, 0, 0] = [1.0, -2.0, 0.5, 0.0]
    vp1[0, 0, 0] = [2.0, -1.0, 4.0]
    q1 = np.array([[[1.0, 1.0, 2.0, 9.0]]], np.float32)
    sink = np.array([0.75], np.float32)
    out = oracle.paged_decode(q1, "f32", kp1, "f32", vp1, "f32", np.array([[0]]), np.array([1]),
                              num_q_heads=1, num_kv_heads=1, head_dim_qk=4, head_dim_v=3,
                              block_size=B, scale=0.5, sinks=sink)
    s0 = 0.5 * (1.0 - 2.0 + 1.0)
    want = vp1[0, 0, 0] / (1.0 + np.exp(0.75 - s0))
    assert np.allclose(out[0, 0], want, rtol=1e-7, atol=1e-7)


def test_window_and_sinks_together_and_empty_sequences():
    lay = W.layout(2, num_seqs=3, len_hi=100)
    lay.seq_lens[:] = [0, 100, 33]
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 3)
    sinks = W.normal(2, 78, (32,))
    got = _run(q, kp, "bf16", vp, "bf16", lay, 32, 8, 0.1, sliding_window=20, sinks=sinks)
    ref = _brute(q, kp, vp, lay, 32, 8, 0.1, window=20, sinks=sinks)
    assert (got[0] == 0).all()
    assert _rel(got[1:], ref[1:]) < 1e-6
