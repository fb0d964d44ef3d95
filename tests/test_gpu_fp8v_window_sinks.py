"""GPU parity of the E4M3 V cache (writes and decode), the sliding window and
attention sinks, against the CPU oracle.

Bars: the E4M3 V store is bit-exact (both sides round fl32(v / v_scale) to
nearest even with saturation); attention within 2e-3 row-relative (FP32
output); bit-identity where an invariant demands it (a sink of -inf, table
entries before the window)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, dev, host, say

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- E4M3 V store

def _v_store_both(v, in_dt, slots, H, D, nblk, v_scale, stride=None):
    ref = np.full((nblk, 16, H, D), 0x5A, np.uint8)
    oracle.cache_write_v(v, in_dt, slots, ref, num_kv_heads=H, head_dim_v=D, block_size=16,
                         cache_dtype="fp8", v_scale=v_scale, in_token_stride=stride)
    pool = dev(np.full((nblk, 16, H, D), 0x5A, np.uint8))
    vt = dev(v)
    if stride is not None:
        vt = vt[:, :H * D].reshape(v.shape[0], H, D)   # strided view of the padded rows
    else:
        vt = vt.reshape(v.shape[0], H, D)
    pkv.cache_write_v(vt, dev(slots), pool, v_scale=v_scale)
    return host(pool), ref


def test_e4m3_v_population_write_whole_pool_bit_exact():
    lay = W.layout(3, num_seqs=6, len_hi=3000)
    start, cu, _ = W.positions_all(lay)
    T = int(cu[-1])
    slots = oracle.fill_slots(lay.block_tables, start, cu, T, 16)
    slots[::11] = -1                                   # padding tokens
    slots[5] = lay.num_blocks * 16 + 3                 # past the pool: skipped
    v = W.kv_tokens(3, T, "v")
    vs = float(np.abs(oracle.to_f64(v, "bf16")).max()) / 448.0 * 0.75   # some saturation
    say(f"E4M3 V population write: T={T} blocks={lay.num_blocks} v_scale={vs:.6g}")
    got, ref = _v_store_both(v, "bf16", slots, 8, 128, lay.num_blocks, vs)
    assert (got == ref).all()


@pytest.mark.parametrize("v_scale", [1.0, 0.0364877, 3.0, 31.999998092651367, 2.0 ** -64,
                                     2.0 ** 64, 2.0 ** -126, 2.0 ** -130, 2.0 ** 127])
def test_e4m3_v_store_every_bf16_pattern_bit_exact(v_scale):
    """All 65536 BF16 patterns (NaN, +-inf, -0, subnormals, saturation) as V
    input, 64 tokens of 8 x 128.  31.999998... = 32 (1 - 2^-24) has an
    all-ones significand, where a reciprocal multiply with one correction
    step from the hardware's approximate reciprocal is not the correctly
    rounded quotient (-4096 / it is -128.00002 in FP32).  2^-64 and 2^64 are
    the ends of the scales whose quotient comes from the host's correctly
    rounded reciprocal and one residual correction; 2^-126, 2^-130 (a
    subnormal) and 2^127 take the full division."""
    pats = np.arange(65536, dtype=np.uint16).reshape(64, 8, 128)
    slots = np.random.default_rng(9).permutation(64).astype(np.int64)
    say(f"E4M3 V store of every BF16 pattern, v_scale={v_scale}")
    got, ref = _v_store_both(pats, "bf16", slots, 8, 128, 4, v_scale)
    assert (got == ref).all()


def test_e4m3_v_store_fp32_strided_input_bit_exact():
    T, H, D = 37, 4, 64
    stride = H * D + 64
    v = W.normal(4, 84, (T, stride)) * 50.0
    v[3, 7] = np.inf
    v[4, 9] = -np.nan
    v[5, 1] = -0.0
    slots = np.random.default_rng(3).permutation(48)[:T].astype(np.int64)
    say(f"E4M3 V store from strided FP32 rows: T={T} H={H} D={D}")
    got, ref = _v_store_both(v, "f32", slots, H, D, 3, 0.37, stride=stride)
    assert (got == ref).all()


@pytest.mark.parametrize("in_dt,H,D", [("bf16", 6, 128), ("bf16", 40, 128), ("f32", 3, 112),
                                        ("f32", 24, 192)])
def test_e4m3_v_store_row_shapes(in_dt, H, D):
    """Rows whose 16-byte output columns do not divide a work-group (48 and 21
    columns: tokens side by side with idle threads) or exceed it (320 and 288
    columns: a column loop), from BF16 and FP32 input, with padding slots."""
    T = 300
    v = W.normal(4, 91 + H, (T, H * D)) * 30.0
    if in_dt == "bf16":
        v = W.bf16_bits(v)
    slots = np.random.default_rng(H + D).permutation(20 * 16)[:T].astype(np.int64)
    slots[::13] = -1
    say(f"E4M3 V store of {in_dt} rows: H={H} D={D}")
    got, ref = _v_store_both(v.reshape(T, H, D), in_dt, slots, H, D, 20, 0.37)
    assert (got == ref).all()


# ---------------------------------------------------------------- decode

def _decode_both(q, q_dt, kp, k_dt, vp, v_dt, lay, *, Hq, Hkv, scale, k_scale=1.0, v_scale=1.0,
                 window=0, sinks=None, split_tokens=0, gate=None):
    Dqk, Dv = kp.shape[-1], vp.shape[-1]
    ref = oracle.paged_decode(q, q_dt, kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                              num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=Dqk, head_dim_v=Dv,
                              block_size=16, scale=scale, k_scale=k_scale, v_scale=v_scale,
                              sliding_window=window, sinks=sinks, gate=gate, nthreads=8)
    say(f"decode S={lay.num_seqs} tokens={lay.total_tokens} Hq={Hq} Hkv={Hkv} D={Dqk}/{Dv} "
        f"K={k_dt} V={v_dt} window={window} sinks={sinks is not None} split={split_tokens}")
    out = pkv.paged_decode_attn(dev(q), dev(kp), dev(vp), dev(lay.block_tables),
                                dev(lay.seq_lens), scale=scale, k_scale=k_scale,
                                v_scale=v_scale, sliding_window=window,
                                sinks=None if sinks is None else dev(sinks),
                                gate=None if gate is None else dev(gate),
                                split_tokens=split_tokens)
    return host(out), ref


def _pools(lay, Hkv, D, k_dt, v_dt, seed):
    rng = np.random.default_rng(seed)
    shape = (lay.num_blocks, 16, Hkv, D)

    def make(dt, stream):
        if dt == "fp8":
            return W.e4m3_codes(2, stream, shape)
        x = rng.standard_normal(shape).astype(np.float32)
        return W.bf16_bits(x) if dt == "bf16" else x
    kp, vp = make(k_dt, seed), make(v_dt, seed + 1)
    for p in (kp, vp):
        p[lay.pad_block] = {np.uint8: 0x7F, np.uint16: 0x7FC0}.get(p.dtype.type, np.nan)
    return kp, vp


@pytest.mark.parametrize("k_dt", ["bf16", "fp8"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_e4m3_v_decode_ragged(k_dt, D, G):
    lay = W.layout_for(2, [1, 15, 16, 17, 333, 700])
    Hkv = 2
    kp, vp = _pools(lay, Hkv, D, k_dt, "fp8", 500 + D + G)
    q = W.bf16_bits(np.random.default_rng(G).standard_normal((6, Hkv * G, D)).astype(np.float32))
    got, ref = _decode_both(q, "bf16", kp, k_dt, vp, "fp8", lay, Hq=Hkv * G, Hkv=Hkv,
                            scale=D ** -0.5, k_scale=0.5, v_scale=0.0625 * 3, split_tokens=128)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


def test_e4m3_kv_decode_workload_subset_with_splits():
    lay = W.layout(3, num_seqs=3, len_hi=20000)
    kp, vp = W.random_pools(3, lay, v_dtype="fp8")
    q = W.queries(3, 3)
    for split in (0, 256):
        got, ref = _decode_both(q, "bf16", kp, "fp8", vp, "fp8", lay, Hq=64, Hkv=8,
                                scale=128 ** -0.5, k_scale=0.25, v_scale=0.02,
                                split_tokens=split)
        err = attn_err(got, ref)
        say(f"  err {err:.3e}")
        assert err <= ATTN_TOL


@pytest.mark.parametrize("window", [1, 5, 16, 17, 100, 1000, 5000])
@pytest.mark.parametrize("split_tokens", [0, 16, 64])
def test_window_mfma_path(window, split_tokens):
    lay = W.layout_for(2, [1, 15, 16, 17, 100, 333, 1500, 4000])
    kp, vp = _pools(lay, 8, 128, "bf16", "bf16", 31)
    q = W.queries(2, lay.num_seqs)
    got, ref = _decode_both(q, "bf16", kp, "bf16", vp, "bf16", lay, Hq=32, Hkv=8,
                            scale=128 ** -0.5, window=window, split_tokens=split_tokens)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("split_tokens", [0, 16, 128])
def test_sinks_mfma_path_with_and_without_window(split_tokens):
    lay = W.layout_for(2, [0, 1, 17, 300, 2500])
    kp, vp = _pools(lay, 8, 128, "bf16", "bf16", 41)
    q = W.queries(2, lay.num_seqs)
    sinks = W.normal(2, 79, (32,)) * 4.0
    for window in (0, 40):
        got, ref = _decode_both(q, "bf16", kp, "bf16", vp, "bf16", lay, Hq=32, Hkv=8,
                                scale=128 ** -0.5, window=window, sinks=sinks,
                                split_tokens=split_tokens)
        err = attn_err(got, ref)
        say(f"  err {err:.3e}")
        assert (got[0] == 0).all() and np.isfinite(got).all() and err <= ATTN_TOL


def test_window_sinks_fp32_path():
    lay = W.layout_for(4, [1, 30, 200, 900])
    Hq = Hkv = 8
    rng = np.random.default_rng(51)
    kp = rng.standard_normal((lay.num_blocks, 16, Hkv, 192)).astype(np.float32)
    vp = rng.standard_normal((lay.num_blocks, 16, Hkv, 128)).astype(np.float32)
    kp[lay.pad_block] = np.nan
    vp[lay.pad_block] = np.nan
    q = rng.standard_normal((lay.num_seqs, Hq, 192)).astype(np.float32)
    sinks = rng.standard_normal(Hq).astype(np.float32)
    for window, split in ((0, 0), (25, 0), (25, 16), (300, 64)):
        got, ref = _decode_both(q, "f32", kp, "f32", vp, "f32", lay, Hq=Hq, Hkv=Hkv,
                                scale=192 ** -0.5, window=window, sinks=sinks,
                                split_tokens=split)
        err = attn_err(got, ref)
        say(f"  err {err:.3e}")
        assert np.isfinite(got).all() and err <= ATTN_TOL


def test_sink_minus_inf_is_bit_identical_to_no_sink():
    lay = W.layout_for(2, [5, 300, 1200])
    kp, vp = _pools(lay, 8, 128, "bf16", "bf16", 61)
    q = W.queries(2, lay.num_seqs)
    args = (dev(q), dev(kp), dev(vp), dev(lay.block_tables), dev(lay.seq_lens))
    for split in (0, 32):
        say(f"sink -inf vs none, split={split}")
        a = host(pkv.paged_decode_attn(*args, scale=0.1, split_tokens=split))
        b = host(pkv.paged_decode_attn(*args, scale=0.1, split_tokens=split,
                                       sinks=dev(np.full(32, -np.inf, np.float32))))
        assert a.tobytes() == b.tobytes()


def test_table_entries_before_the_window_are_never_read():
    lay = W.layout_for(2, [700, 1300])
    kp, vp = _pools(lay, 8, 128, "bf16", "bf16", 71)
    q = W.queries(2, lay.num_seqs)
    bt = lay.block_tables.copy()
    bt[0, :(700 - 64) // 16] = 2 ** 30
    bt[1, :(1300 - 64) // 16] = -3
    args = (dev(q), dev(kp), dev(vp))
    say("window 64 with garbage table entries before the window")
    a = host(pkv.paged_decode_attn(*args, dev(lay.block_tables), dev(lay.seq_lens), scale=0.1,
                                   sliding_window=64, split_tokens=16))
    b = host(pkv.paged_decode_attn(*args, dev(bt), dev(lay.seq_lens), scale=0.1,
                                   sliding_window=64, split_tokens=16))
    assert a.tobytes() == b.tobytes()
