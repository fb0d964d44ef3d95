"""Pins of the oracle's paged decode attention.

The oracle is checked against: contiguous attention built from numpy matmul
and scipy's softmax on KV gathered through the block table (a library
routine, no paging); closed forms (seq_len 1 returns V; q = 0 or equal keys
give the mean of V; two tokens give a logistic mix); invariants (block-table
permutation, GQA equals MHA with repeated KV heads, gate 1 and 0); and the
degenerate cases (seq_len 0, tokens of unmapped blocks).
Page 1 (kv_cache.rs, doc of paged_decode_attn_fp8) fixes the inputs:
block_tables i32 [num_seqs * max_blocks_per_seq], seq_lens i32, num_q_heads /
num_kv_heads, inv_sqrt_d, k_scale; page 3 (mla_cuda.rs) the optional gate.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import pkv_workloads as W


def gather_contiguous(pool, dtype, bt, n, B, scl=1.0):
    """[n, H, D] FP64 rows of one sequence, via the block table."""
    rows = pool.reshape(-1, *pool.shape[2:])
    idx = np.array([bt[t // B] * B + t % B for t in range(n)], np.int64)
    x = oracle.to_f64(rows[idx], dtype)
    return x * scl if dtype == "fp8" else x


def brute(q, q_dt, kp, k_dt, vp, v_dt, bt, lens, Hq, Hkv, B, scale, k_scale=1.0, gate=None):
    S = len(lens)
    G = Hq // Hkv
    out = np.zeros((S, Hq, vp.shape[-1]))
    qf = oracle.to_f64(q, q_dt)
    for s in range(S):
        n = int(lens[s])
        if n <= 0:
            continue
        K = gather_contiguous(kp, k_dt, bt[s], n, B, k_scale)
        V = gather_contiguous(vp, v_dt, bt[s], n, B)
        for h in range(Hq):
            sc = scale * (K[:, h // G, :] @ qf[s, h])
            out[s, h] = softmax(sc) @ V[:, h // G, :]
    if gate is not None:
        out = out * gate
    return out


def run(q, q_dt, kp, k_dt, vp, v_dt, lay, Hq, Hkv, scale, **kw):
    return oracle.paged_decode(q, q_dt, kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                               num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=kp.shape[-1],
                               head_dim_v=vp.shape[-1], block_size=lay.block_size,
                               scale=scale, **kw)


def rel_err(got, ref):
    den = np.abs(ref).max(axis=-1, keepdims=True)
    return float((np.abs(got - ref) / np.maximum(den, 1e-300)).max())


def test_tiny_workload_matches_brute_force():
    lay = W.layout(0)
    kp, vp = W.random_pools(0, lay)
    q = W.queries(0, 1)
    got = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 4, 2, 0.125)
    ref = brute(q, "bf16", kp, "bf16", vp, "bf16", lay.block_tables, lay.seq_lens, 4, 2, 16,
                0.125)
    assert rel_err(got, ref) < 1e-6


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_groups_partial_blocks_match_brute_force(G):
    lay = W.layout(2, num_seqs=5, len_hi=300)          # ragged lengths, partial last blocks
    lay.seq_lens[:] = [1, 17, 250, 300, 33]
    Hkv = 8
    kp, vp = W.random_pools(2, lay)
    q = W.normal(2, 90 + G, (5, Hkv * G, 128))
    q = W.bf16_bits(q)
    got = run(q, "bf16", kp, "bf16", vp, "bf16", lay, Hkv * G, Hkv, 128 ** -0.5)
    ref = brute(q, "bf16", kp, "bf16", vp, "bf16", lay.block_tables, lay.seq_lens, Hkv * G,
                Hkv, 16, 128 ** -0.5)
    assert rel_err(got, ref) < 1e-6


def test_fp8_k_matches_brute_force_with_scale():
    lay = W.layout(3, num_seqs=3, len_hi=200)
    kp, vp = W.random_pools(3, lay)
    q = W.queries(3, 3)
    ks = 0.25
    got = run(q, "bf16", kp, "fp8", vp, "bf16", lay, 64, 8, 128 ** -0.5, k_scale=ks)
    ref = brute(q, "bf16", kp, "fp8", vp, "bf16", lay.block_tables, lay.seq_lens, 64, 8, 16,
                128 ** -0.5, k_scale=ks)
    assert rel_err(got, ref) < 1e-6
    # k_scale enters exactly as a factor on the scores
    got2 = run(q, "bf16", kp, "fp8", vp, "bf16", lay, 64, 8, 128 ** -0.5 * 2, k_scale=ks / 2)
    assert rel_err(got2, got) < 1e-6


def test_f32_mha_dqk_ne_dv_with_gate_matches_brute_force():
    lay = W.layout(4, len_hi=96)
    kp = W.normal(4, 91, (lay.num_blocks, 16, 4, 192))
    vp = W.normal(4, 92, (lay.num_blocks, 16, 4, 128))
    q = W.normal(4, 93, (1, 4, 192))
    g = W.uniform(4, 94, (1, 4, 128), 0.0, 1.0)
    got = run(q, "f32", kp, "f32", vp, "f32", lay, 4, 4, 192 ** -0.5, gate=g)
    ref = brute(q, "f32", kp, "f32", vp, "f32", lay.block_tables, lay.seq_lens, 4, 4, 16,
                192 ** -0.5, gate=g)
    assert rel_err(got, ref) < 1e-6


def test_q_rope_prologue_equals_rotating_q_first():
    """The decode's q rotation at position n-1 equals writing q through the
    K path's RoPE (no norm) at that position, then attending unrotated."""
    lay = W.layout(4, len_hi=64)
    H, Dqk, Dv = 2, 192, 128
    kp = W.normal(4, 95, (lay.num_blocks, 16, H, Dqk))
    vp = W.normal(4, 96, (lay.num_blocks, 16, H, Dv))
    q = W.normal(4, 97, (1, H, Dqk))
    n = int(lay.seq_lens[0])
    kw = dict(q_rope_theta=50000.0, q_rope_offset=128, q_rope_dim=64)
    a = run(q, "f32", kp, "f32", vp, "f32", lay, H, H, 0.1, q_rope=True, **kw)
    cache = np.zeros((1, 16, H, Dqk), np.float32)
    oracle.cache_write_k(q, "f32", np.array([0], np.int64), cache, "f32", num_kv_heads=H,
                         head_dim=Dqk, block_size=16, pos_t=np.array([n - 1]), theta=50000.0,
                         rope_offset=128, rotary_dim=64)
    qr = cache[0, 0][None]
    b = run(qr, "f32", kp, "f32", vp, "f32", lay, H, H, 0.1)
    assert rel_err(a, b) < 1e-6


def test_seq_len_one_returns_v_row_exactly():
    lay = W.layout(2, num_seqs=4, len_hi=64)
    lay.seq_lens[:] = 1
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 4)
    got = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 128 ** -0.5)
    rows = vp.reshape(-1, 8, 128)
    for s in range(4):
        v0 = oracle.f32_from_bf16(rows[lay.block_tables[s, 0] * 16])
        assert (got[s] == np.repeat(v0, 4, axis=0)).all()


def test_zero_query_and_equal_keys_give_mean_of_v():
    lay = W.layout(2, num_seqs=2, len_hi=100)
    kp, vp = W.random_pools(2, lay)
    q0 = np.zeros((2, 32, 128), np.uint16)                 # +0.0 in BF16
    got = run(q0, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    kp_eq = np.broadcast_to(kp[lay.block_tables[0, 0], 0], kp.shape).copy()
    q = W.queries(2, 2)
    got2 = run(q, "bf16", kp_eq, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    for s in range(2):
        n = int(lay.seq_lens[s])
        V = gather_contiguous(vp, "bf16", lay.block_tables[s], n, 16)
        mean = V.mean(axis=0)                              # [Hkv, Dv]
        want = np.repeat(mean, 4, axis=0)
        assert rel_err(got[s], want) < 1e-6
        assert rel_err(got2[s], want) < 1e-6


def test_two_tokens_logistic_mix():
    """n = 2: out = sigma(s1 - s2) v1 + sigma(s2 - s1) v2 with s_t = scale q.k_t."""
    B = 16
    kp = np.zeros((1, B, 1, 4), np.float32)
    vp = np.zeros((1, B, 1, 3), np.float32)
    kp[0, 0, 0] = [1.0, 0.0, 0.0, 0.0]
    kp[0, 1, 0] = [0.0, 2.0, 0.0, 0.0]
    vp[0, 0, 0] = [1.0, 0.0, 5.0]
    vp[0, 1, 0] = [0.0, 1.0, -5.0]
    q = np.array([[[3.0, 1.0, 0.0, 7.0]]], np.float32)
    out = oracle.paged_decode(q, "f32", kp, "f32", vp, "f32", np.array([[0]]), np.array([2]),
                              num_q_heads=1, num_kv_heads=1, head_dim_qk=4, head_dim_v=3,
                              block_size=B, scale=0.5)
    s1, s2 = 0.5 * 3.0, 0.5 * 2.0
    a = 1.0 / (1.0 + np.exp(s2 - s1))
    want = a * vp[0, 0, 0] + (1 - a) * vp[0, 1, 0]
    assert np.allclose(out[0, 0], want, rtol=1e-7, atol=1e-7)


def test_block_table_permutation_invariance():
    lay = W.layout(2, num_seqs=3, len_hi=160)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 3)
    a = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    perm = np.random.default_rng(5).permutation(lay.num_blocks)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    lay2 = W.Layout(lay.index, lay.seq_lens, perm[lay.block_tables].astype(np.int32),
                    lay.num_blocks, int(perm[lay.pad_block]), 16)
    b = run(q, "bf16", kp2, "bf16", vp2, "bf16", lay2, 32, 8, 0.1)
    assert a.tobytes() == b.tobytes()


def test_gqa_equals_mha_with_repeated_kv_heads():
    lay = W.layout(2, num_seqs=2, len_hi=80)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 2)
    a = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    kr = np.repeat(kp, 4, axis=2)
    vr = np.repeat(vp, 4, axis=2)
    b = run(q, "bf16", kr, "bf16", vr, "bf16", lay, 32, 32, 0.1)
    assert a.tobytes() == b.tobytes()


def test_gate_one_and_zero():
    lay = W.layout(2, num_seqs=2, len_hi=80)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 2)
    a = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    one = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1,
              gate=np.ones((2, 32, 128), np.float32))
    zero = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1,
               gate=np.zeros((2, 32, 128), np.float32))
    assert a.tobytes() == one.tobytes()
    assert (zero == 0).all()


def test_empty_sequences_and_unmapped_blocks():
    lay = W.layout(2, num_seqs=3, len_hi=64)
    lay.seq_lens[:] = [0, 40, 40]
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 3)
    out = run(q, "bf16", kp, "bf16", vp, "bf16", lay, 32, 8, 0.1)
    assert (out[0] == 0).all()
    # an unmapped (negative) block id excludes its tokens: same as a sequence
    # holding only the other blocks' tokens
    bt = lay.block_tables.copy()
    bt[2, 0] = -1
    lay2 = W.Layout(2, lay.seq_lens, bt, lay.num_blocks, lay.pad_block, 16)
    masked = run(q, "bf16", kp, "bf16", vp, "bf16", lay2, 32, 8, 0.1)
    ref = brute(q[2:3], "bf16", kp, "bf16", vp, "bf16",
                np.array([list(bt[2, 1:3]) + [0]]), np.array([24]), 32, 8, 16, 0.1)
    # tokens 16..39 of sequence 2 are tokens 0..23 of the shifted table
    assert rel_err(masked[2:3], ref) < 1e-6
    assert np.isfinite(out).all()
