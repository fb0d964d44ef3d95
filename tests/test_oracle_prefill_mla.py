"""Pins of the oracle's paged prefill attention and MLA cache assembly.

Prefill (page 1 names batched N-token variants of the paged kernels; the
reading pinned here is causal attention over the same cache: the q_len
queries of a sequence are its last q_len tokens, query i at position
p = seq_len - q_len + i attends to [lo, p]): checked against numpy/scipy
causal attention over the gathered rows, closed forms (a fresh sequence's
first query returns v_0), invariants (q_len 1 is decode; rows after p do not
change query p; one chunk equals two consecutive chunks; window and sinks as
for decode).

MLA cache assembly (page 1, mla_cache_assemble: [kv_latent | k_rope] -> K,
[kv_latent | zeros] -> V): byte equality of both rows, padding slots skipped,
other rows untouched.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle
import pkv_workloads as W


def _gather(pool, dt, bt, n, scl=1.0):
    rows = pool.reshape(-1, *pool.shape[2:])
    idx = np.array([bt[t // 16] * 16 + t % 16 for t in range(n)], np.int64)
    x = oracle.to_f64(rows[idx], dt)
    return x * scl if dt == "fp8" else x


def _case(qlens, lens, Hq=8, Hkv=2, D=64, seed=0):
    lay = W.layout_for(2, lens)
    rng = np.random.default_rng(seed)
    kp = W.bf16_bits(rng.standard_normal((lay.num_blocks, 16, Hkv, D)).astype(np.float32))
    vp = W.bf16_bits(rng.standard_normal((lay.num_blocks, 16, Hkv, D)).astype(np.float32))
    kp[lay.pad_block] = 0x7FC0
    vp[lay.pad_block] = 0x7FC0
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = W.bf16_bits(rng.standard_normal((int(cu[-1]), Hq, D)).astype(np.float32))
    return lay, kp, vp, cu, q


def _prefill(q, cu, kp, vp, lay, Hq, Hkv, scale, **kw):
    return oracle.paged_prefill(q, "bf16", cu, kp, "bf16", vp, "bf16", lay.block_tables,
                                lay.seq_lens, num_q_heads=Hq, num_kv_heads=Hkv,
                                head_dim_qk=kp.shape[-1], head_dim_v=vp.shape[-1], block_size=16,
                                scale=scale, **kw)


def _brute(q, cu, kp, vp, lay, Hq, Hkv, scale, window=0, sinks=None):
    G = Hq // Hkv
    out = np.zeros((q.shape[0], Hq, vp.shape[-1]))
    qf = oracle.to_f64(q, "bf16")
    for s in range(len(lay.seq_lens)):
        n = int(lay.seq_lens[s])
        K = _gather(kp, "bf16", lay.block_tables[s], n)
        V = _gather(vp, "bf16", lay.block_tables[s], n)
        qlen = int(cu[s + 1] - cu[s])
        for i in range(qlen):
            p = n - qlen + i
            lo = p + 1 - window if 0 < window < p + 1 else 0
            for h in range(Hq):
                sc = scale * (K[lo:p + 1, h // G, :] @ qf[cu[s] + i, h])
                w = softmax(np.append(sc, sinks[h]))[:-1] if sinks is not None else softmax(sc)
                out[cu[s] + i, h] = w @ V[lo:p + 1, h // G, :]
    return out


def _rel(got, ref):
    den = np.abs(ref).max(axis=-1, keepdims=True)
    return float((np.abs(got - ref) / np.maximum(den, 1e-300)).max())


def test_prefill_matches_causal_brute_force():
    lay, kp, vp, cu, q = _case([5, 1, 40, 17], [70, 1, 40, 200])
    got = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125)
    ref = _brute(q, cu, kp, vp, lay, 8, 2, 0.125)
    assert np.isfinite(got).all() and _rel(got, ref) < 1e-6


@pytest.mark.parametrize("window", [1, 7, 16, 33])
def test_prefill_window_and_sinks_match_brute_force(window):
    lay, kp, vp, cu, q = _case([20, 3, 64], [90, 3, 64], seed=window)
    sinks = W.normal(2, 80, (8,))
    got = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125, sliding_window=window, sinks=sinks)
    ref = _brute(q, cu, kp, vp, lay, 8, 2, 0.125, window=window, sinks=sinks)
    assert _rel(got, ref) < 1e-6


def test_fresh_sequence_first_query_returns_first_v_row():
    lay, kp, vp, cu, q = _case([30], [30])
    got = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125)
    v0 = oracle.f32_from_bf16(vp.reshape(-1, 2, 64)[lay.block_tables[0, 0] * 16])
    assert (got[0] == np.repeat(v0, 4, axis=0)).all()


def test_q_len_one_is_decode():
    lay, kp, vp, cu, q = _case([1, 1, 1], [1, 77, 300])
    got = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125, sliding_window=50)
    dec = oracle.paged_decode(q, "bf16", kp, "bf16", vp, "bf16", lay.block_tables, lay.seq_lens,
                              num_q_heads=8, num_kv_heads=2, head_dim_qk=64, head_dim_v=64,
                              block_size=16, scale=0.125, sliding_window=50)
    assert got.tobytes() == dec.tobytes()


def test_rows_after_a_query_do_not_change_it():
    lay, kp, vp, cu, q = _case([24], [100])
    a = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125)
    # overwrite the K/V rows of positions 90..99 (queries 14..23 see them)
    kp2, vp2 = kp.copy(), vp.copy()
    for t in range(90, 100):
        blk = lay.block_tables[0, t // 16]
        kp2[blk, t % 16] = 0x4000
        vp2[blk, t % 16] = 0xC000
    b = _prefill(q, cu, kp2, vp2, lay, 8, 2, 0.125)
    first = 90 - (100 - 24)                       # query index of position 90
    assert a[:first].tobytes() == b[:first].tobytes()
    assert not np.array_equal(a[first:], b[first:])


def test_one_chunk_equals_two_consecutive_chunks():
    lay, kp, vp, cu, q = _case([40], [120])
    whole = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125)
    L1 = 25
    lay1 = W.Layout(lay.index, np.array([120 - 40 + L1], np.int32), lay.block_tables,
                    lay.num_blocks, lay.pad_block, 16)
    first = _prefill(q[:L1], np.array([0, L1], np.int32), kp, vp, lay1, 8, 2, 0.125)
    second = _prefill(q[L1:], np.array([0, 40 - L1], np.int32), kp, vp, lay, 8, 2, 0.125)
    assert np.concatenate([first, second]).tobytes() == whole.tobytes()


def test_queries_before_position_zero_and_empty_sequences():
    lay, kp, vp, cu, q = _case([0, 5, 3], [10, 3, 0])
    got = _prefill(q, cu, kp, vp, lay, 8, 2, 0.125)
    # sequence 1 has 3 tokens but 5 queries: the first two sit before position 0
    assert (got[0:2] == 0).all() and (got[5:8] == 0).all()
    ref = _brute(q[2:5], np.array([0, 0, 3, 3], np.int32), kp, vp, lay, 8, 2, 0.125)
    assert _rel(got[2:5], ref) < 1e-6


# ---------------------------------------------------------------- MLA assembly

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mla_cache_assemble_rows(dtype):
    T, lora, rope, dim = 9, 64, 16, 96            # row longer than lora + rope: zero tail
    rng = np.random.default_rng(4)
    lat = rng.standard_normal((T, lora + 8)).astype(np.float32)   # strided rows
    kr = rng.standard_normal((T, rope)).astype(np.float32)
    if dtype == "bf16":
        lat, kr = W.bf16_bits(lat), W.bf16_bits(kr)
    npt = lat.dtype
    kc = np.full((2, 16, 1, dim), 7, npt)
    vc = np.full((2, 16, 1, dim), 7, npt)
    slots = np.array([3, -1, 31, 0, 64, 17, 18, 5, 6], np.int64)
    oracle.mla_cache_assemble(lat, kr, dtype, slots, kc, vc, kv_lora=lora, rope=rope,
                              block_size=16, latent_stride=lora + 8)
    K = kc.reshape(-1, dim)
    V = vc.reshape(-1, dim)
    for t, s in enumerate(slots):
        if not 0 <= s < 32:
            continue
        assert (K[s, :lora] == lat[t, :lora]).all() and (K[s, lora:lora + rope] == kr[t]).all()
        assert (K[s, lora + rope:] == 0).all()
        assert (V[s, :lora] == lat[t, :lora]).all() and (V[s, lora:] == 0).all()
    untouched = np.setdiff1d(np.arange(32), slots[(slots >= 0) & (slots < 32)])
    assert (K[untouched] == 7).all() and (V[untouched] == 7).all()
