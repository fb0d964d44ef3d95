"""GPU parity of paged prefill attention and MLA cache assembly against the
CPU oracle.

Bars: attention within 2e-3 row-relative (FP32 output); the MLA rows
bit-exact (whole pools, sentinel-filled, compared byte for byte)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, dev, host, say

pytestmark = pytest.mark.gpu


def _pools(lay, Hkv, D, k_dt, v_dt, seed):
    rng = np.random.default_rng(seed)
    shape = (lay.num_blocks, 16, Hkv, D)

    def make(dt, stream):
        if dt == "fp8":
            return W.e4m3_codes(2, stream, shape)
        return W.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    kp, vp = make(k_dt, seed), make(v_dt, seed + 1)
    for p in (kp, vp):
        p[lay.pad_block] = 0x7F if p.dtype == np.uint8 else 0x7FC0
    return kp, vp


def _both(qlens, lens, *, Hq, Hkv, D, k_dt="bf16", v_dt="bf16", seed=0, k_scale=1.0,
          v_scale=1.0, window=0, sinks=None, max_q_len=None):
    lay = W.layout_for(2, lens)
    kp, vp = _pools(lay, Hkv, D, k_dt, v_dt, seed)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(cu[-1])
    q = W.bf16_bits(np.random.default_rng(seed + 7).standard_normal((T, Hq, D)).astype(np.float32))
    scale = D ** -0.5
    ref = oracle.paged_prefill(q, "bf16", cu, kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                               num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D,
                               block_size=16, scale=scale, k_scale=k_scale, v_scale=v_scale,
                               sliding_window=window, sinks=sinks, nthreads=8)
    mql = int(max(qlens)) if max_q_len is None else max_q_len
    say(f"prefill q_lens={list(qlens)[:6]} lens={list(lens)[:6]} Hq={Hq} Hkv={Hkv} D={D} "
        f"K={k_dt} V={v_dt} window={window} sinks={sinks is not None}")
    out = pkv.paged_prefill_attn(dev(q), dev(cu), dev(kp), dev(vp), dev(lay.block_tables),
                                 dev(lay.seq_lens), max_q_len=mql, scale=scale, k_scale=k_scale,
                                 v_scale=v_scale, sliding_window=window,
                                 sinks=None if sinks is None else dev(sinks))
    return host(out), ref


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_gqa_ragged(G, D):
    got, ref = _both([1, 17, 64, 5, 0, 33], [1, 17, 300, 900, 40, 33], Hq=2 * G, Hkv=2, D=D,
                     seed=G + D)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("k_dt,v_dt", [("fp8", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")])
def test_prefill_e4m3_caches(k_dt, v_dt):
    got, ref = _both([40, 100, 7], [500, 100, 2000], Hq=32, Hkv=8, D=128, k_dt=k_dt, v_dt=v_dt,
                     seed=11, k_scale=0.5, v_scale=0.1875)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("window", [1, 16, 50, 700])
def test_prefill_window_and_sinks(window):
    sinks = W.normal(2, 81, (32,)) * 2.0
    got, ref = _both([64, 130, 3], [64, 1000, 3], Hq=32, Hkv=8, D=128, seed=window,
                     window=window, sinks=sinks)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


def test_prefill_queries_before_position_zero_and_short_max_q_len():
    # sequence 0: 9 queries over 4 tokens (5 rows at p < 0 are zero)
    got, ref = _both([9, 20], [4, 50], Hq=8, Hkv=2, D=64, seed=3)
    assert (got[:5] == 0).all()
    assert attn_err(got, ref) <= ATTN_TOL
    # max_q_len below a sequence's q_len: its first max_q_len rows are still right
    # (rows past them are left undefined by the contract)
    got2, _ = _both([9, 20], [4, 50], Hq=8, Hkv=2, D=64, seed=3, max_q_len=9)
    assert attn_err(got2[:9 + 9], ref[:9 + 9]) <= ATTN_TOL


def test_prefill_workload_subset():
    lay = W.layout(2, num_seqs=6)
    qlens = np.minimum(lay.seq_lens, 96)
    got, ref = _both(qlens, lay.seq_lens, Hq=32, Hkv=8, D=128, seed=5)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert err <= ATTN_TOL


def test_chunked_prefill_chain_through_the_writes():
    """fill_slots -> K write -> V write of the new chunk, then prefill, on the
    GPU and in the oracle, over a pool already holding the earlier tokens."""
    lay = W.layout(1, num_seqs=4)
    cfg = lay.cfg
    H, Hq, D = cfg["num_kv_heads"], cfg["num_q_heads"], cfg["head_dim"]
    lens = lay.seq_lens.astype(np.int64)
    qlens = np.minimum(lens, 70).astype(np.int32)
    start = (lens - qlens).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    T = int(cu[-1])
    kp, vp = _pools(lay, H, D, "bf16", "bf16", 21)
    k = W.kv_tokens(1, T, "k")
    v = W.kv_tokens(1, T, "v")
    w = W.norm_weight(1)
    pos = np.concatenate([np.arange(s, s + n) for s, n in zip(start, qlens)]).astype(np.int32)
    q = W.bf16_bits(np.random.default_rng(22).standard_normal((T, Hq, D)).astype(np.float32))
    slots = oracle.fill_slots(lay.block_tables, start, cu, T, 16)
    kr, vr = kp.copy(), vp.copy()
    oracle.cache_write_k(k, "bf16", slots, kr, "bf16", num_kv_heads=H, head_dim=D,
                         block_size=16, norm_weight=w, eps=cfg["eps"], pos_t=pos,
                         theta=cfg["theta"])
    oracle.cache_write_v(v, "bf16", slots, vr, num_kv_heads=H, head_dim_v=D, block_size=16)
    ref = oracle.paged_prefill(q, "bf16", cu, kr, "bf16", vr, "bf16", lay.block_tables,
                               lay.seq_lens, num_q_heads=Hq, num_kv_heads=H, head_dim_qk=D,
                               head_dim_v=D, block_size=16, scale=D ** -0.5, nthreads=8)
    say(f"chunked prefill chain: T={T} Hq={Hq} Hkv={H}")
    bt = dev(lay.block_tables)
    sd = torch.empty(T, dtype=torch.int64, device="cuda")
    pkv.fill_slots(sd, bt, dev(start), dev(cu), 16)
    kc, vc = dev(kp), dev(vp)
    pkv.cache_write_k_fused(dev(k), sd, kc, norm_weight=dev(w), eps=cfg["eps"], pos_t=dev(pos),
                            theta=cfg["theta"])
    pkv.cache_write_v(dev(v), sd, vc)
    out = pkv.paged_prefill_attn(dev(q), dev(cu), kc, vc, bt, dev(lay.seq_lens),
                                 max_q_len=int(qlens.max()), scale=D ** -0.5)
    err = attn_err(host(out), ref)
    say(f"  err {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_mla_cache_assemble_bit_exact(dtype):
    T, lora, rope, dim = 300, 512, 64, 576 + (16 if dtype == "f32" else 0)
    rng = np.random.default_rng(31)
    lat = rng.standard_normal((T, lora + 32)).astype(np.float32)
    kr = rng.standard_normal((T, rope)).astype(np.float32)
    if dtype == "bf16":
        lat, kr = W.bf16_bits(lat), W.bf16_bits(kr)
    nb = 24
    slots = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots[::13] = -1
    slots[7] = nb * 16 + 5
    sentinel = np.full((nb, 16, 1, dim), 0x3F if dtype == "f32" else 0x5A5A, lat.dtype)
    kref, vref = sentinel.copy(), sentinel.copy()
    oracle.mla_cache_assemble(lat, kr, dtype, slots, kref, vref, kv_lora=lora, rope=rope,
                              block_size=16, latent_stride=lora + 32)
    say(f"MLA cache assembly {dtype}: T={T} lora={lora} rope={rope} dim={dim}")
    kc, vc = dev(sentinel), dev(sentinel)
    latd = dev(lat)
    pkv.mla_cache_assemble(latd[:, :lora], dev(kr), dev(slots), kc, vc, kv_lora=lora, rope=rope)
    assert host(kc).tobytes() == kref.tobytes()
    assert host(vc).tobytes() == vref.tobytes()


@pytest.mark.parametrize("Hkv", [1, 3, 5])
@pytest.mark.parametrize("G", [1, 8])
def test_prefill_kv_head_counts(Hkv, G):
    got, ref = _both([1, 40, 130], [1, 300, 700], Hq=Hkv * G, Hkv=Hkv, D=128, seed=Hkv + G,
                     k_dt="fp8" if Hkv == 3 else "bf16", k_scale=0.5)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL
