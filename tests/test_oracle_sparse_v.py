"""Pins of the oracle's sparse-V decode (oracle.paged_decode_sparse_v).

Page 2 (kv_cache_fp8k.rs, paged_decode_attn_fp8k_turbo3v) skips the V load
and dequantisation of a position whose attention weight is at most a
threshold, and page 1 describes its Turbo-V decodes as sparse in V; the
threshold's value is not given.  The oracle returns the sum of w_t v_t over the positions
with w_t > tau and, as ``bound``, the sum of w_t |v_t| over the others.

Pinned against: the exact decode (tau = 0, itself pinned in
test_oracle_decode.py); hand-worked two-token and sink cases whose weights
are 1/4, 3/4 or exactly 1/2 (the "at most" boundary); scipy's softmax for
the kept mass of a constant V; and the bracket exact - bound <= out <=
exact + bound for any V.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import pkv_workloads as W


def sparse(q, kp, vp, lay, Hq, Hkv, scale, tau, k_dt="bf16", v_dt="bf16", **kw):
    return oracle.paged_decode_sparse_v(q, "bf16", kp, k_dt, vp, v_dt, lay.block_tables,
                                        lay.seq_lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                        head_dim_qk=kp.shape[-1], head_dim_v=128 if
                                        v_dt.startswith("tq") else vp.shape[-1],
                                        block_size=16, scale=scale, tau=tau, nthreads=8, **kw)


def exact(q, kp, vp, lay, Hq, Hkv, scale, k_dt="bf16", v_dt="bf16", **kw):
    return oracle.paged_decode(q, "bf16", kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                               num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=kp.shape[-1],
                               head_dim_v=128 if v_dt.startswith("tq") else vp.shape[-1],
                               block_size=16, scale=scale, nthreads=8, **kw)


def one_seq(n, H=1, D=16):
    """A one-sequence layout of n tokens; pools [blocks, 16, H, D] of zeros."""
    lay = W.layout_for(2, [n])
    shape = (lay.num_blocks, 16, H, D)
    return lay, np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)


def put(pool, lay, t, row):
    """Row of token t (kv head 0) of the only sequence, as BF16."""
    blk = lay.block_tables[0, t // 16]
    pool[blk, t % 16, 0, :] = W.bf16_bits(np.asarray(row, np.float32))


def bf(x):
    return oracle.to_f64(W.bf16_bits(np.asarray(x, np.float32)), "bf16")


@pytest.mark.parametrize("case", ["bf16", "fp8k_window_sinks_gate", "tq3", "tq2_window"])
def test_tau_zero_is_the_exact_decode(case):
    lay = W.layout_for(2, [0, 1, 15, 17, 300, 999])
    Hkv, G, D = 2, 4, 128
    Hq = Hkv * G
    q = W.bf16_bits(W.normal(2, 300, (lay.num_seqs, Hq, D)))
    kw, k_dt, v_dt, ks = {}, "bf16", "bf16", 1.0
    if case.startswith("fp8k"):
        k_dt, ks = "fp8", 0.5
        kp = W.e4m3_finite_codes(2, 301, (lay.num_blocks, 16, Hkv, D))
        kw = dict(sliding_window=40, sinks=W.normal(2, 302, (Hq,)) * 3,
                  gate=W.normal(2, 303, (lay.num_seqs, Hq, D)))
    else:
        kp = W.bf16_bits(W.normal(2, 304, (lay.num_blocks, 16, Hkv, D)))
    if case.startswith("tq"):
        bits = int(case[2])
        v_dt = f"tq{bits}"
        vp = np.zeros((lay.num_blocks, oracle.tq_block_bytes(bits, 16, Hkv, D)), np.uint8)
        x = W.normal(2, 305, (lay.num_blocks * 16, Hkv, D))
        oracle.cache_write_v(x, "f32", np.arange(lay.num_blocks * 16, dtype=np.int64), vp,
                             num_kv_heads=Hkv, head_dim_v=D, block_size=16, cache_dtype=v_dt)
        if case.endswith("window"):
            kw = dict(sliding_window=100)
    else:
        vp = W.bf16_bits(W.normal(2, 306, (lay.num_blocks, 16, Hkv, D)))
    out, bound = sparse(q, kp, vp, lay, Hq, Hkv, D ** -0.5, 0.0, k_dt, v_dt, k_scale=ks, **kw)
    ref = exact(q, kp, vp, lay, Hq, Hkv, D ** -0.5, k_dt, v_dt, k_scale=ks, **kw)
    assert (bound == 0).all()
    np.testing.assert_allclose(out, ref, rtol=1e-6, atol=1e-7)
    assert (out[0] == 0).all()                        # empty sequence: zero row


def test_two_tokens_weights_one_quarter_three_quarters():
    """Scores 0 and ln 3 (q = e0, k1 = e0, scale = ln 3): weights 1/4, 3/4."""
    lay, kp, vp = one_seq(2)
    put(kp, lay, 1, np.eye(16)[0])
    v0 = W.normal(2, 310, (16,))
    v1 = W.normal(2, 311, (16,))
    put(vp, lay, 0, v0)
    put(vp, lay, 1, v1)
    q = W.bf16_bits(np.eye(16, dtype=np.float32)[0].reshape(1, 1, 16))
    scale = float(np.float32(math.log(3.0)))
    a, b = bf(v0), bf(v1)
    for tau, want, want_bound in ((0.1, 0.25 * a + 0.75 * b, 0 * a),
                                  (0.3, 0.75 * b, 0.25 * np.abs(a)),
                                  (0.8, 0 * a, 0.25 * np.abs(a) + 0.75 * np.abs(b))):
        out, bound = sparse(q, kp, vp, lay, 1, 1, scale, tau)
        np.testing.assert_allclose(out[0, 0], want, atol=1e-6)
        np.testing.assert_allclose(bound[0, 0], want_bound, atol=1e-6)


def test_a_weight_equal_to_the_threshold_is_skipped():
    """Equal scores give weights of exactly 1/2: skipped at tau = 1/2, kept
    just below it."""
    lay, kp, vp = one_seq(2)
    v0, v1 = W.normal(2, 312, (16,)), W.normal(2, 313, (16,))
    put(vp, lay, 0, v0)
    put(vp, lay, 1, v1)
    q = W.bf16_bits(W.normal(2, 314, (1, 1, 16)))   # all keys 0: equal scores
    a, b = bf(v0), bf(v1)
    out, bound = sparse(q, kp, vp, lay, 1, 1, 0.25, 0.5)
    assert (out == 0).all()
    assert (bound[0, 0] == (0.5 * np.abs(a) + 0.5 * np.abs(b)).astype(np.float32)).all()
    out, bound = sparse(q, kp, vp, lay, 1, 1, 0.25, float(np.nextafter(0.5, 0.0)))
    assert (out[0, 0] == (0.5 * a + 0.5 * b).astype(np.float32)).all()
    assert (bound == 0).all()


def test_the_sink_joins_the_denominator():
    """One token of score 0 and a sink logit of 0: the token's weight is 1/2."""
    lay, kp, vp = one_seq(1)
    v0 = W.normal(2, 315, (16,))
    put(vp, lay, 0, v0)
    q = W.bf16_bits(W.normal(2, 316, (1, 1, 16)))
    sinks = np.zeros(1, np.float32)
    a = bf(v0)
    out, bound = sparse(q, kp, vp, lay, 1, 1, 0.25, 0.5, sinks=sinks)
    assert (out == 0).all() and (bound[0, 0] == (0.5 * np.abs(a)).astype(np.float32)).all()
    out, bound = sparse(q, kp, vp, lay, 1, 1, 0.25, 0.4, sinks=sinks)
    assert (out[0, 0] == (0.5 * a).astype(np.float32)).all() and (bound == 0).all()


@pytest.mark.parametrize("tau", [1e-4, 1e-3, 1e-2, 0.05])
def test_constant_v_kept_mass_matches_scipy_softmax(tau):
    """V = c everywhere: out = c times the softmax mass above tau, out + bound
    = c; the kept mass from scipy's softmax over the gathered scores."""
    n, D, c = 200, 64, 1.5
    lay = W.layout_for(2, [n])
    k = W.bf16_bits(W.normal(2, 320, (lay.num_blocks, 16, 1, D)) * 2.0)
    v = np.full((lay.num_blocks, 16, 1, D), W.bf16_bits(np.float32(c)), np.uint16)
    q = W.bf16_bits(W.normal(2, 321, (1, 1, D)))
    out, bound = sparse(q, k, v, lay, 1, 1, D ** -0.5, tau)
    rows = oracle.to_f64(k, "bf16").reshape(-1, D)
    idx = [lay.block_tables[0, t // 16] * 16 + t % 16 for t in range(n)]
    w = softmax(D ** -0.5 * (rows[idx] @ oracle.to_f64(q, "bf16")[0, 0]))
    kept = w[w > tau].sum()
    assert 0 < kept < 1                                # both sides occur
    np.testing.assert_allclose(out[0, 0], c * kept, rtol=1e-6)
    np.testing.assert_allclose(out[0, 0] + bound[0, 0], c, rtol=1e-6)


@pytest.mark.parametrize("tau", [1e-3, 2e-2])
def test_exact_output_lies_within_the_bound(tau):
    """|exact - out| <= bound elementwise, with peaked weights (large scores)
    and a gate; the gate multiplies out and |gate| the bound."""
    lay = W.layout_for(2, [5, 100, 513])
    Hkv, G, D = 2, 2, 64
    q = W.bf16_bits(W.normal(2, 330, (3, Hkv * G, D)) * 4.0)
    kp = W.bf16_bits(W.normal(2, 331, (lay.num_blocks, 16, Hkv, D)))
    vp = W.bf16_bits(W.normal(2, 332, (lay.num_blocks, 16, Hkv, D)))
    gate = W.normal(2, 333, (3, Hkv * G, D))
    out, bound = sparse(q, kp, vp, lay, Hkv * G, Hkv, D ** -0.5, tau)
    ref = exact(q, kp, vp, lay, Hkv * G, Hkv, D ** -0.5)
    assert (bound > 0).any()
    assert (np.abs(ref - out) <= bound + 1e-6).all()
    gout, gbound = sparse(q, kp, vp, lay, Hkv * G, Hkv, D ** -0.5, tau, gate=gate)
    np.testing.assert_allclose(gout, out * gate, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(gbound, bound * np.abs(gate), rtol=1e-6, atol=1e-7)
