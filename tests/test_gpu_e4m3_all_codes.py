"""Decode and prefill over E4M3 K and V pools holding every finite E4M3 code
(magnitude codes 0x00..0x7E with both signs: subnormals, every exponent
field up to 448), on both paths that widen the codes in registers
(v_cvt_scalef32_pk_bf16_fp8 for K, v_cvt_scalef32_pk_f16_fp8 for V), against
the oracle.  Bar: 2e-3 row-relative (FP32 output)."""
import numpy as np
import pytest

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, dev, host, say

pytestmark = pytest.mark.gpu

K_SCALE = 2.0 ** -8          # |k| <= 1.75: scores of N(0,1) queries stay moderate
V_SCALE = 2.0 ** -6


def _pools(lay, Hkv, D, k_dt, v_dt, seed):
    shape = (lay.num_blocks, 16, Hkv, D)

    def make(dt, stream):
        if dt == "fp8":
            p = W.e4m3_finite_codes(2, stream, shape)
            seen = np.unique(p)
            assert seen.size == 254, seen.size               # all finite codes, both signs
            return p
        return W.bf16_bits(np.random.default_rng(stream).standard_normal(shape).astype(np.float32))
    kp, vp = make(k_dt, seed), make(v_dt, seed + 1)
    for p in (kp, vp):
        p[lay.pad_block] = 0x7F if p.dtype == np.uint8 else 0x7FC0
    return kp, vp


@pytest.mark.parametrize("k_dt,v_dt", [("fp8", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")])
@pytest.mark.parametrize("G,D", [(1, 128), (4, 128), (8, 128), (8, 64)])
def test_decode_every_e4m3_code(k_dt, v_dt, G, D):
    Hkv = 4
    lay = W.layout_for(2, [1, 16, 17, 250, 777, 2048, 3001])
    kp, vp = _pools(lay, Hkv, D, k_dt, v_dt, 300 + G + D)
    q = W.bf16_bits(np.random.default_rng(G).standard_normal(
        (lay.num_seqs, Hkv * G, D)).astype(np.float32))
    ks = K_SCALE if k_dt == "fp8" else 1.0
    vs = V_SCALE if v_dt == "fp8" else 1.0
    ref = oracle.paged_decode(q, "bf16", kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                              num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim_qk=D,
                              head_dim_v=D, block_size=16, scale=D ** -0.5, k_scale=ks,
                              v_scale=vs, nthreads=8)
    for split in (0, 64):
        say(f"decode over every E4M3 code: K={k_dt} V={v_dt} G={G} D={D} split={split}")
        out = pkv.paged_decode_attn(dev(q), dev(kp), dev(vp), dev(lay.block_tables),
                                    dev(lay.seq_lens), scale=D ** -0.5, k_scale=ks, v_scale=vs,
                                    split_tokens=split)
        got = host(out)
        err = attn_err(got, ref)
        say(f"  err {err:.3e}")
        assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("k_dt,v_dt", [("fp8", "bf16"), ("bf16", "fp8"), ("fp8", "fp8")])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_prefill_every_e4m3_code(k_dt, v_dt, G):
    Hkv, D = 2, 128
    lens = [40, 300, 1200]
    qlens = [40, 129, 64]
    lay = W.layout_for(2, lens)
    kp, vp = _pools(lay, Hkv, D, k_dt, v_dt, 400 + G)
    cu = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = W.bf16_bits(np.random.default_rng(G + 1).standard_normal(
        (int(cu[-1]), Hkv * G, D)).astype(np.float32))
    ks = K_SCALE if k_dt == "fp8" else 1.0
    vs = V_SCALE if v_dt == "fp8" else 1.0
    ref = oracle.paged_prefill(q, "bf16", cu, kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                               num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D,
                               block_size=16, scale=D ** -0.5, k_scale=ks, v_scale=vs, nthreads=8)
    say(f"prefill over every E4M3 code: K={k_dt} V={v_dt} G={G}")
    out = pkv.paged_prefill_attn(dev(q), dev(cu), dev(kp), dev(vp), dev(lay.block_tables),
                                 dev(lay.seq_lens), max_q_len=max(qlens), scale=D ** -0.5,
                                 k_scale=ks, v_scale=vs)
    got = host(out)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL
