"""GPU parity of the TurboQuant-style V cache (b = 2, 3, 4 bits per code, one
E4M3 scale per 16 elements): the write kernel and the decode attention that
reads it, against the CPU oracle.

Bars: the oracle takes the encoder's decisions (codes, E4M3 scale bytes) in
FP64 from the definition and the kernel in FP32, so the written pool is
compared tie-aware: codes and scale bytes equal except where the FP64
decision lies within FP32 rounding of its boundary (there one step apart at
most), bytes outside the written slots untouched; attention within 2e-3
row-relative (FP32 output), as for the other caches."""
import os

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import (ATTN_TOL, attn_err, dev, host, say, tq_compare, tq_rows_by_slot,
                   tq_scale_mask, tq_written_mask)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _blk(bits, H, D):
    return oracle.tq_block_bytes(bits, 16, H, D)


def _write_both(v, in_dt, slots, H, D, nblk, bits, stride=None):
    """The same rows written by the oracle and by the library into pools
    pre-filled with 0x5A; returns (gpu pool, oracle pool)."""
    ref = np.full((nblk, _blk(bits, H, D)), 0x5A, np.uint8)
    oracle.cache_write_v(v, in_dt, slots, ref, num_kv_heads=H, head_dim_v=D, block_size=16,
                         cache_dtype=f"tq{bits}", in_token_stride=stride)
    pool = dev(np.full((nblk, _blk(bits, H, D)), 0x5A, np.uint8), torch.uint8)
    vt = dev(v)
    vt = (vt[:, :H * D] if stride is not None else vt).reshape(v.shape[0], H, D)
    pkv.cache_write_v(vt, dev(slots), pool, tq_bits=bits)
    return host(pool), ref


def _check_write(got, ref, v, in_dt, slots, H, D, bits, stride=None):
    """Bytes outside the written slots untouched; the written slots' codes
    and scales tie-aware against the oracle's FP64 encoder."""
    keep = (slots >= 0) & (slots < got.shape[0] * 16)
    written = tq_written_mask(got.shape[0], bits, H, D, slots[keep])
    assert (got[~written] == ref[~written]).all(), "bytes outside the written slots changed"
    gc, gs = tq_rows_by_slot(got, slots[keep], bits, H, D)
    st = tq_compare(gc, gs, v[keep], in_dt, bits, H, D, in_token_stride=stride)
    say(f"  {st}")
    return st


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_tq_population_write(bits):
    lay = W.layout(3, num_seqs=6, len_hi=3000)
    start, cu, _ = W.positions_all(lay)
    T = int(cu[-1])
    slots = oracle.fill_slots(lay.block_tables, start, cu, T, 16)
    slots[::11] = -1                                   # padding tokens
    slots[5] = lay.num_blocks * 16 + 3                 # past the pool: skipped
    v = W.kv_tokens(3, T, "v")
    say(f"TQ{bits} V population write: T={T} blocks={lay.num_blocks}")
    got, ref = _write_both(v, "bf16", slots, 8, 128, lay.num_blocks, bits)
    st = _check_write(got, ref, v, "bf16", slots, 8, 128, bits)
    assert st["groups_out_of_fp32_range"] == 0


def _special_rows(T, H, D, seed):
    """FP32 rows of varied magnitude with zero groups, -0, single-element
    groups and ties of the decision rule."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((T, H, D)) *
         np.exp(rng.uniform(-8, 8, (T, H, 1)))).astype(np.float32)
    x[1, 0, :16] = 0.0                                 # all-zero group
    x[1, 0, 16:32] = -0.0                              # all -0 group
    x[2, 1, 3] = -0.0
    x[3, 0, 16:32] = 0.0
    x[3, 0, 20] = -5.0                                 # one non-zero element
    ties = [0.5, -1.0625, 1.8125] + [1.0] * 9 + [1.5, 0.1875, 0.1875, 0.125]
    x[4, 1, :16] = np.array(ties, np.float32)
    x[5, 0, :16] = np.float32(0.75) * np.sign(rng.standard_normal(16)).astype(np.float32)
    return x


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_tq_write_fp32_strided_special_groups(bits):
    T, H, D = 37, 4, 64
    stride = H * D + 64
    x = _special_rows(T, H, D, bits)
    v = np.zeros((T, stride), np.float32)
    v[:, :H * D] = x.reshape(T, -1)
    v[:, H * D:] = np.nan                              # never read
    slots = np.random.default_rng(3).permutation(48)[:T].astype(np.int64)
    say(f"TQ{bits} V write from strided FP32 rows: T={T} H={H} D={D}")
    got, ref = _write_both(v, "f32", slots, H, D, 3, bits, stride=stride)
    _check_write(got, ref, v, "f32", slots, H, D, bits, stride=stride)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_tq_write_extreme_magnitudes(bits):
    """Groups whose sum of squares is subnormal, underflows to 0, or
    overflows to infinity in FP32 (BF16 input spans the whole FP32 range):
    their scale bytes (0, or saturated at 448) equal the definition's; codes
    are compared only where the FP32 sum of squares is a normal number."""
    T, H, D = 8, 2, 32
    rng = np.random.default_rng(40 + bits)
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    x[0] *= np.float32(1e-21)                          # squares subnormal
    x[1] *= np.float32(1e-24)                          # squares underflow to 0
    x[2] *= np.float32(1e20)                           # sum overflows to inf
    x[3, 0, :16] = 0.0
    x[3, 0, 7] = np.float32(3e38)
    x[4] *= np.float32(1e-19)
    v = W.bf16_bits(x)
    slots = np.arange(T, dtype=np.int64)[::-1].copy()
    say(f"TQ{bits} V write of extreme magnitudes")
    got, ref = _write_both(v, "bf16", slots, H, D, 1, bits)
    st = _check_write(got, ref, v, "bf16", slots, H, D, bits)
    assert st["groups_out_of_fp32_range"] > 0


def test_tq3_write_of_the_hand_worked_ties_group():
    rows = {}
    for line in open(os.path.join(GOLDEN, "tq3_ties_example.txt")):
        if line.strip() and not line.startswith("#"):
            k, *val = line.split()
            rows[k] = val
    x = np.array([float(a) for a in rows["x"]], np.float32).reshape(1, 1, 16)
    pool = dev(np.zeros((1, _blk(3, 1, 16)), np.uint8), torch.uint8)
    say("TQ3 write of the ties example")
    pkv.cache_write_v(dev(x), dev(np.zeros(1, np.int64)), pool, tq_bits=3)
    got = host(pool)[0]
    assert bytes(got[:6]) == bytes(int(b, 16) for b in rows["bytes"])
    assert got[16 * 6] == int(rows["scale"][0], 16)


# ---------------------------------------------------------------- decode

def _tq_pool(lay, H, D, bits, seed, random_codes=False):
    """A TQ V pool over every slot: rows of varied magnitude encoded by the
    oracle, or random code bytes with random finite scales; the padding
    block's scales are NaN (0x7F), so a read of it would show."""
    nb = lay.num_blocks
    blk = _blk(bits, H, D)
    sm = tq_scale_mask(bits, H, D)
    pool = np.zeros((nb, blk), np.uint8)
    if random_codes:
        pool[:, ~sm] = np.random.default_rng(seed).integers(0, 256, (nb, int((~sm).sum())),
                                                             dtype=np.uint8)
        pool[:, sm] = W.e4m3_codes(2, seed, (nb, int(sm.sum())))
    else:
        rng = np.random.default_rng(seed)
        x = (rng.standard_normal((nb * 16, H, D)) *
             np.exp(rng.uniform(-2, 2, (nb * 16, H, 1)))).astype(np.float32)
        oracle.cache_write_v(x, "f32", np.arange(nb * 16, dtype=np.int64), pool, num_kv_heads=H,
                             head_dim_v=D, block_size=16, cache_dtype=f"tq{bits}")
    if lay.pad_block >= 0:
        pool[lay.pad_block, sm] = 0x7F
    return pool


def _k_pool(lay, H, D, k_dt, seed):
    shape = (lay.num_blocks, 16, H, D)
    if k_dt == "fp8":
        kp = W.e4m3_codes(2, seed, shape)
        kp[lay.pad_block] = 0x7F
    else:
        kp = W.bf16_bits(np.random.default_rng(seed).standard_normal(shape).astype(np.float32))
        kp[lay.pad_block] = 0x7FC0
    return kp


def _decode_both(q, kp, k_dt, vp, bits, lay, *, Hq, Hkv, scale, k_scale=1.0, window=0,
                 sinks=None, split_tokens=0):
    D = kp.shape[-1]
    ref = oracle.paged_decode(q, "bf16", kp, k_dt, vp, f"tq{bits}", lay.block_tables,
                              lay.seq_lens, num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D,
                              head_dim_v=D, block_size=16, scale=scale, k_scale=k_scale,
                              sliding_window=window, sinks=sinks, nthreads=8)
    say(f"decode TQ{bits} V: S={lay.num_seqs} tokens={lay.total_tokens} Hq={Hq} Hkv={Hkv} "
        f"K={k_dt} window={window} sinks={sinks is not None} split={split_tokens}")
    out = pkv.paged_decode_attn(dev(q), dev(kp), dev(vp, torch.uint8), dev(lay.block_tables),
                                dev(lay.seq_lens), scale=scale, k_scale=k_scale,
                                sliding_window=window,
                                sinks=None if sinks is None else dev(sinks),
                                split_tokens=split_tokens, v_tq_bits=bits)
    return host(out), ref


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("k_dt", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_tq_decode_ragged(bits, k_dt, G):
    lay = W.layout_for(2, [1, 15, 16, 17, 333, 700])
    Hkv, D = 2, 128
    kp = _k_pool(lay, Hkv, D, k_dt, 600 + G)
    vp = _tq_pool(lay, Hkv, D, bits, 700 + bits + G)
    q = W.bf16_bits(np.random.default_rng(G).standard_normal((6, Hkv * G, D)).astype(np.float32))
    got, ref = _decode_both(q, kp, k_dt, vp, bits, lay, Hq=Hkv * G, Hkv=Hkv, scale=D ** -0.5,
                            k_scale=0.5, split_tokens=128)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_tq_decode_every_code_value(bits):
    """Random code bytes: every code of the format, with random scales."""
    lay = W.layout_for(2, [5, 64, 130, 999])
    kp = _k_pool(lay, 8, 128, "bf16", 801)
    vp = _tq_pool(lay, 8, 128, bits, 802 + bits, random_codes=True)
    q = W.queries(2, lay.num_seqs)
    got, ref = _decode_both(q, kp, "bf16", vp, bits, lay, Hq=32, Hkv=8, scale=128 ** -0.5,
                            split_tokens=64)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


def test_tq3_decode_workload_subset_with_splits():
    lay = W.layout(3, num_seqs=3, len_hi=20000)
    kp = _k_pool(lay, 8, 128, "fp8", 811)
    vp = _tq_pool(lay, 8, 128, 3, 812)
    q = W.queries(3, 3)
    for split in (0, 256):
        got, ref = _decode_both(q, kp, "fp8", vp, 3, lay, Hq=64, Hkv=8, scale=128 ** -0.5,
                                k_scale=0.25, split_tokens=split)
        err = attn_err(got, ref)
        say(f"  err {err:.3e}")
        assert err <= ATTN_TOL


@pytest.mark.parametrize("bits", [2, 4])
def test_tq_decode_window_and_sinks(bits):
    lay = W.layout_for(2, [0, 1, 17, 300, 2500])
    kp = _k_pool(lay, 8, 128, "bf16", 821)
    vp = _tq_pool(lay, 8, 128, bits, 822)
    q = W.queries(2, lay.num_seqs)
    sinks = W.normal(2, 79, (32,)) * 4.0
    for window, split in ((0, 0), (40, 16), (1000, 128)):
        got, ref = _decode_both(q, kp, "bf16", vp, bits, lay, Hq=32, Hkv=8, scale=128 ** -0.5,
                                window=window, sinks=sinks, split_tokens=split)
        err = attn_err(got, ref)
        say(f"  err {err:.3e}")
        assert (got[0] == 0).all() and np.isfinite(got).all() and err <= ATTN_TOL


def test_tq_write_then_decode_round_trip():
    """The library's own write feeds its decode; the write is held to the
    tie-aware bar, and the oracle decodes the pool the library wrote."""
    lay = W.layout_for(2, [70, 513])
    start, cu, _ = W.positions_all(lay)
    T = int(cu[-1])
    slots = oracle.fill_slots(lay.block_tables, start, cu, T, 16)
    v = W.bf16_bits(W.normal(2, 90, (T, 8, 128)))
    say(f"TQ3 write -> decode round trip: T={T}")
    ref_pool = np.zeros((lay.num_blocks, _blk(3, 8, 128)), np.uint8)
    oracle.cache_write_v(v, "bf16", slots, ref_pool, num_kv_heads=8, head_dim_v=128,
                         block_size=16, cache_dtype="tq3")
    pool = dev(np.zeros_like(ref_pool), torch.uint8)
    pkv.cache_write_v(dev(v), dev(slots), pool, tq_bits=3)
    kp = _k_pool(lay, 8, 128, "bf16", 831)
    q = W.queries(2, lay.num_seqs)
    got = host(pkv.paged_decode_attn(dev(q), dev(kp), pool, dev(lay.block_tables),
                                     dev(lay.seq_lens), scale=128 ** -0.5, v_tq_bits=3))
    gpool = host(pool)
    _check_write(gpool, ref_pool, v, "bf16", slots, 8, 128, 3)
    ref = oracle.paged_decode(q, "bf16", kp, "bf16", gpool, "tq3", lay.block_tables,
                              lay.seq_lens, num_q_heads=32, num_kv_heads=8, head_dim_qk=128,
                              head_dim_v=128, block_size=16, scale=128 ** -0.5, nthreads=8)
    assert attn_err(got, ref) <= ATTN_TOL
