"""GPU parity of paged decode attention against the CPU oracle.

Inputs are seeded pools filled directly with random values (decode tested on
its own; the padding block is NaN so a read of it would show), plus the
end-to-end tiny workload where the pools are written by the GPU write path
and the oracle writes its own.  Bar: max row-relative error <= 2e-3 (FP32
output), bit-identity where an invariant demands it."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, dev, host, say

pytestmark = pytest.mark.gpu


def run_both(index, lay, *, Hq, Hkv, D, Dv=None, q=None, kp=None, vp=None, k_scale=1.0,
             gate=None, split_tokens=0, scale=None, q_rope=False, **rope):
    cfg = W.WORKLOADS[index]
    Dv = D if Dv is None else Dv
    kdt = cfg["k_cache_dtype"]
    vdt = cfg["kv_dtype"]
    qdt = cfg["kv_dtype"]
    if kp is None:
        kp, vp = W.random_pools(index, lay)
    if q is None:
        q = W.queries(index, lay.num_seqs)
    scale = D ** -0.5 if scale is None else scale
    ref = oracle.paged_decode(q, qdt, kp, kdt, vp, vdt, lay.block_tables, lay.seq_lens,
                              num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=Dv,
                              block_size=16, scale=scale, k_scale=k_scale, gate=gate,
                              q_rope=q_rope, nthreads=8, **rope)
    say(f"decode workload {index}: S={lay.num_seqs} tokens={lay.total_tokens} Hq={Hq} "
        f"Hkv={Hkv} D={D}/{Dv} K={kdt} split={split_tokens}")
    out = pkv.paged_decode_attn(dev(q), dev(kp), dev(vp), dev(lay.block_tables),
                                dev(lay.seq_lens), scale=scale, k_scale=k_scale,
                                gate=None if gate is None else dev(gate),
                                split_tokens=split_tokens, q_rope=q_rope, **rope)
    got = host(out)
    return got, ref


def test_tiny_end_to_end_chain():
    """fill_slots -> K write -> V write -> decode on the GPU, against the
    oracle's own chain on the same inputs."""
    lay = W.layout(0)
    cfg = lay.cfg
    H, Hq, D = cfg["num_kv_heads"], cfg["num_q_heads"], cfg["head_dim"]
    start, cu, pos = W.positions_all(lay)
    T = int(cu[-1])
    k, v, w, q = W.kv_tokens(0, T, "k"), W.kv_tokens(0, T, "v"), W.norm_weight(0), W.queries(0, 1)
    s_ref = oracle.fill_slots(lay.block_tables, start, cu, T, 16)
    kc_ref = np.zeros((16, 16, H, D), np.uint16)
    vc_ref = np.zeros((16, 16, H, D), np.uint16)
    oracle.cache_write_k(k, "bf16", s_ref, kc_ref, "bf16", num_kv_heads=H, head_dim=D,
                         block_size=16, norm_weight=w, pos_t=pos)
    oracle.cache_write_v(v, "bf16", s_ref, vc_ref, num_kv_heads=H, head_dim_v=D, block_size=16)
    ref = oracle.paged_decode(q, "bf16", kc_ref, "bf16", vc_ref, "bf16", lay.block_tables,
                              lay.seq_lens, num_q_heads=Hq, num_kv_heads=H, head_dim_qk=D,
                              head_dim_v=D, block_size=16, scale=0.125)
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    bt = dev(lay.block_tables)
    pkv.fill_slots(slots, bt, dev(start.astype(np.int32)), dev(cu.astype(np.int32)), 16)
    kc = torch.zeros((16, 16, H, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    pkv.cache_write_k_fused(dev(k), slots, kc, norm_weight=dev(w), pos_t=dev(pos))
    pkv.cache_write_v(dev(v), slots, vc)
    out = pkv.paged_decode_attn(dev(q), kc, vc, bt, dev(lay.seq_lens), scale=0.125)
    err = attn_err(host(out), ref)
    say(f"  tiny chain attention error {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D", [64, 128])
def test_bf16_gqa_groups_ragged(G, D):
    lay = W.layout_for(2, [1, 15, 16, 17, 333, 700])
    Hkv = 2
    B = 16
    rng = np.random.default_rng(G * 1000 + D)
    kp = W.bf16_bits(rng.standard_normal((lay.num_blocks, B, Hkv, D)).astype(np.float32))
    vp = W.bf16_bits(rng.standard_normal((lay.num_blocks, B, Hkv, D)).astype(np.float32))
    kp[lay.pad_block] = 0x7FC0
    vp[lay.pad_block] = 0x7FC0
    q = W.bf16_bits(rng.standard_normal((6, Hkv * G, D)).astype(np.float32))
    got, ref = run_both(2, lay, Hq=Hkv * G, Hkv=Hkv, D=D, q=q, kp=kp, vp=vp, split_tokens=128)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("case", ["many_short_some_long", "past_balanced_limit", "one_range"])
def test_automatic_plan_modes(case):
    """Automatic split size without a window: up to 1024 sequences take equal
    block ranges over the whole batch (short sequences share a work-group, long
    ones span several ranges and are merged), more sequences take one work-group
    per (sequence, split); a batch small enough for one range needs no
    workspace.  Empty sequences give zero rows in every mode."""
    rng = np.random.default_rng(77)
    if case == "many_short_some_long":
        lens = rng.integers(0, 48, size=600)
        lens[::97] = rng.integers(500, 3000, size=lens[::97].size)
        lens[5] = 0
    elif case == "past_balanced_limit":
        lens = rng.integers(0, 40, size=1100)
        lens[7] = 0
    else:
        lens = np.array([20])
    lay = W.layout_for(2, lens)
    Hkv, G, D, B = 2, 4, 64, 16
    kp = W.bf16_bits(rng.standard_normal((lay.num_blocks, B, Hkv, D)).astype(np.float32))
    vp = W.bf16_bits(rng.standard_normal((lay.num_blocks, B, Hkv, D)).astype(np.float32))
    kp[lay.pad_block] = 0x7FC0
    vp[lay.pad_block] = 0x7FC0
    q = W.bf16_bits(rng.standard_normal((lens.size, Hkv * G, D)).astype(np.float32))
    if case == "one_range":
        assert pkv.decode_workspace_bytes(1, Hkv * G, Hkv, D, lay.max_blocks_per_seq, B) == 0
    got, ref = run_both(2, lay, Hq=Hkv * G, Hkv=Hkv, D=D, q=q, kp=kp, vp=vp)
    err = attn_err(got, ref)
    say(f"  {case}: err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL
    assert (got[lens == 0] == 0).all()


def test_bf16_decode_workload_subset():
    lay = W.layout(2, num_seqs=24)
    got, ref = run_both(2, lay, Hq=32, Hkv=8, D=128)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert err <= ATTN_TOL


def test_fp8k_decode_workload_subset():
    lay = W.layout(3, num_seqs=3, len_hi=20000)
    got, ref = run_both(3, lay, Hq=64, Hkv=8, D=128, k_scale=0.25)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("split_tokens", [16, 64, 256, 1024])
def test_split_size_invariance(split_tokens):
    lay = W.layout(2, num_seqs=4, len_hi=4000)
    got, ref = run_both(2, lay, Hq=32, Hkv=8, D=128, split_tokens=split_tokens)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert err <= ATTN_TOL


def test_seq_len_one_returns_v_exactly():
    lay = W.layout_for(2, [1, 1, 1, 1, 1], max_blocks_per_seq=4)
    kp, vp = W.random_pools(2, lay)
    got, ref = run_both(2, lay, Hq=32, Hkv=8, D=128, kp=kp, vp=vp)
    assert (got == ref).all()


def test_block_table_permutation_bit_identical():
    lay = W.layout(2, num_seqs=4, len_hi=900)
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 4)
    a = pkv.paged_decode_attn(dev(q), dev(kp), dev(vp), dev(lay.block_tables),
                              dev(lay.seq_lens), scale=0.1)
    perm = np.random.default_rng(9).permutation(lay.num_blocks)
    kp2, vp2 = np.empty_like(kp), np.empty_like(vp)
    kp2[perm] = kp
    vp2[perm] = vp
    bt2 = perm[lay.block_tables].astype(np.int32)
    b = pkv.paged_decode_attn(dev(q), dev(kp2), dev(vp2), dev(bt2), dev(lay.seq_lens), scale=0.1)
    assert host(a).tobytes() == host(b).tobytes()


def test_gate_one_zero_and_empty_sequences():
    lay = W.layout_for(2, [0, 300, 5, 0])
    kp, vp = W.random_pools(2, lay)
    q = W.queries(2, 4)
    args = (dev(q), dev(kp), dev(vp), dev(lay.block_tables), dev(lay.seq_lens))
    plain = host(pkv.paged_decode_attn(*args, scale=0.1, split_tokens=64))
    one = host(pkv.paged_decode_attn(*args, scale=0.1, split_tokens=64,
                                     gate=torch.ones((4, 32, 128), device="cuda")))
    zero = host(pkv.paged_decode_attn(*args, scale=0.1, split_tokens=64,
                                      gate=torch.zeros((4, 32, 128), device="cuda")))
    assert plain.tobytes() == one.tobytes()
    assert (zero == 0).all()
    assert (plain[0] == 0).all() and (plain[3] == 0).all()
    ref = oracle.paged_decode(q, "bf16", kp, "bf16", vp, "bf16", lay.block_tables, lay.seq_lens,
                              num_q_heads=32, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                              block_size=16, scale=0.1)
    assert attn_err(plain, ref) <= ATTN_TOL


def test_unmapped_blocks_are_excluded():
    lay = W.layout(2, num_seqs=2, len_hi=200)
    bt = lay.block_tables.copy()
    bt[0, 2] = -1
    bt[1, 0] = lay.num_blocks + 5
    lay2 = W.Layout(2, lay.seq_lens, bt, lay.num_blocks, lay.pad_block, 16)
    got, ref = run_both(2, lay2, Hq=32, Hkv=8, D=128, split_tokens=64)
    assert np.isfinite(got).all() and attn_err(got, ref) <= ATTN_TOL


@pytest.mark.parametrize("q_rope", [False, True])
def test_gated_mla_style_f32_full_size(q_rope):
    """One sequence of 4096, 64 heads (MHA), Dqk 192 / Dv 128, FP32, gate U(0,1),
    query rotated over its last 64 dims at position 4095 unless NoPE."""
    lay = W.layout(4)
    H = 64
    kp = W.normal(4, W.S_POOLK, (lay.num_blocks, 16, H, 192))
    vp = W.normal(4, W.S_POOLV, (lay.num_blocks, 16, H, 128))
    q = W.queries(4, 1)
    g = W.gate(4, 1)
    got, ref = run_both(4, lay, Hq=H, Hkv=H, D=192, Dv=128, q=q, kp=kp, vp=vp, gate=g,
                        q_rope=q_rope, q_rope_theta=50000.0, q_rope_offset=128, q_rope_dim=64)
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert err <= ATTN_TOL


@pytest.mark.parametrize("G", [1, 4, 8])
def test_f32_gqa_groups(G):
    lay = W.layout(4, len_hi=500)
    Hkv = 2
    rng = np.random.default_rng(G)
    kp = rng.standard_normal((lay.num_blocks, 16, Hkv, 128)).astype(np.float32)
    vp = rng.standard_normal((lay.num_blocks, 16, Hkv, 64)).astype(np.float32)
    q = rng.standard_normal((1, Hkv * G, 128)).astype(np.float32)
    got, ref = run_both(4, lay, Hq=Hkv * G, Hkv=Hkv, D=128, Dv=64, q=q, kp=kp, vp=vp,
                        split_tokens=128)
    assert attn_err(got, ref) <= ATTN_TOL


@pytest.mark.parametrize("Hkv", [1, 3, 5])
@pytest.mark.parametrize("G", [1, 16])
@pytest.mark.parametrize("kv", ["bf16/bf16", "fp8/bf16", "bf16/fp8", "bf16/tq3"])
def test_kv_head_counts(Hkv, G, kv):
    """One kv head (MQA) and odd counts, which pack one wavefront per
    work-group, for every MFMA-path cache format."""
    k_dt, v_dt = kv.split("/")
    D = 128
    lay = W.layout_for(2, [1, 40, 300, 1000])
    rng = np.random.default_rng(Hkv * 100 + G)
    shape = (lay.num_blocks, 16, Hkv, D)
    kp = W.e4m3_codes(2, 40 + Hkv, shape) if k_dt == "fp8" else \
        W.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    if v_dt == "tq3":
        vp = np.zeros((lay.num_blocks, oracle.tq_block_bytes(3, 16, Hkv, D)), np.uint8)
        x = rng.standard_normal((lay.num_blocks * 16, Hkv, D)).astype(np.float32)
        oracle.cache_write_v(x, "f32", np.arange(lay.num_blocks * 16, dtype=np.int64), vp,
                             num_kv_heads=Hkv, head_dim_v=D, block_size=16, cache_dtype="tq3")
    elif v_dt == "fp8":
        vp = W.e4m3_codes(2, 50 + Hkv, shape)
    else:
        vp = W.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    q = W.bf16_bits(rng.standard_normal((4, Hkv * G, D)).astype(np.float32))
    ref = oracle.paged_decode(q, "bf16", kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                              num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D,
                              block_size=16, scale=D ** -0.5, k_scale=0.5, v_scale=0.25,
                              nthreads=8)
    say(f"decode Hkv={Hkv} G={G} K={k_dt} V={v_dt}")
    vdev = dev(vp, torch.uint8) if v_dt == "tq3" else dev(vp)
    out = pkv.paged_decode_attn(dev(q), dev(kp), vdev, dev(lay.block_tables), dev(lay.seq_lens),
                                scale=D ** -0.5, k_scale=0.5, v_scale=0.25, split_tokens=256,
                                v_tq_bits=3 if v_dt == "tq3" else 0)
    err = attn_err(host(out), ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(host(out)).all() and err <= ATTN_TOL


@pytest.mark.parametrize("kv", ["bf16/bf16", "fp8/bf16", "bf16/fp8", "bf16/tq3"])
def test_balanced_plan_formats_gate_and_many_pieces(kv):
    """The balanced plan (automatic split size, no window) for every MFMA-path
    cache format, with an output gate: 8 ragged sequences get ranges of a single
    block, so a long sequence is merged from hundreds of partial rows; gate = 1
    is bit-identical to no gate."""
    k_dt, v_dt = kv.split("/")
    Hkv, G, D = 2, 4, 128
    lens = [0, 1, 40, 300, 1000, 2500, 17, 5000]
    lay = W.layout_for(2, lens)
    rng = np.random.default_rng(len(kv) * 7 + ord(kv[0]))
    shape = (lay.num_blocks, 16, Hkv, D)
    kp = W.e4m3_codes(2, 60, shape) if k_dt == "fp8" else \
        W.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    if v_dt == "tq3":
        vp = np.zeros((lay.num_blocks, oracle.tq_block_bytes(3, 16, Hkv, D)), np.uint8)
        x = rng.standard_normal((lay.num_blocks * 16, Hkv, D)).astype(np.float32)
        oracle.cache_write_v(x, "f32", np.arange(lay.num_blocks * 16, dtype=np.int64), vp,
                             num_kv_heads=Hkv, head_dim_v=D, block_size=16, cache_dtype="tq3")
    elif v_dt == "fp8":
        vp = W.e4m3_codes(2, 61, shape)
    else:
        vp = W.bf16_bits(rng.standard_normal(shape).astype(np.float32))
    q = W.bf16_bits(rng.standard_normal((len(lens), Hkv * G, D)).astype(np.float32))
    gate = rng.uniform(0.0, 1.0, (len(lens), Hkv * G, D)).astype(np.float32)
    ref = oracle.paged_decode(q, "bf16", kp, k_dt, vp, v_dt, lay.block_tables, lay.seq_lens,
                              num_q_heads=Hkv * G, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D,
                              block_size=16, scale=D ** -0.5, k_scale=0.5, v_scale=0.25,
                              gate=gate, nthreads=8)
    say(f"balanced plan K={k_dt} V={v_dt} lens={lens}")
    vdev = dev(vp, torch.uint8) if v_dt == "tq3" else dev(vp)
    args = (dev(q), dev(kp), vdev, dev(lay.block_tables), dev(lay.seq_lens))
    kw = dict(scale=D ** -0.5, k_scale=0.5, v_scale=0.25, v_tq_bits=3 if v_dt == "tq3" else 0)
    got = host(pkv.paged_decode_attn(*args, gate=dev(gate), **kw))
    err = attn_err(got, ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL
    assert (got[0] == 0).all()
    plain = host(pkv.paged_decode_attn(*args, **kw))
    ones = host(pkv.paged_decode_attn(*args, gate=dev(np.ones_like(gate)), **kw))
    assert plain.tobytes() == ones.tobytes()
