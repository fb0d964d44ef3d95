"""GPU parity at the full workload sizes, in the launch configuration that
bench.py times, checked on sampled outputs the oracle computes one by one.

Each decode workload is built as the bench builds it: every sequence's
history (n - 1 tokens) goes through the library's slot fill, fused K write
and V write into the shuffled pools; then one decode step writes the new
token of every sequence and runs the decode attention over the whole batch
with the automatic split plan.  Checked against the oracle:
  * slots of the decode step: all of them, bit-exact;
  * K rows of sampled history tokens and of the new tokens of sampled
    sequences: the K-store bar (BF16 <= 1 ulp or the row floor, E4M3 <= 1
    step); V rows of the same tokens bit-exact (copy, E4M3 or TQ bytes);
  * the attention output of sampled sequences (the shortest, the longest and
    random ones), recomputed by the oracle over the blocks those sequences
    own (gathered from the device pools): <= 2e-3 row-relative; with the
    sparse-V skip (heavy keys written into the pool, as the bench does),
    within the oracle's bound of its sparse-V output plus 2e-3.
The prefill workload is checked the same way on sampled sequences.
"""
import numpy as np
import pytest
import torch

import bench
import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, bf16_ok, e4m3_ok, host, say, tq_compare, tq_rows_by_slot

pytestmark = pytest.mark.gpu

B = 16
V_SCALE = 0.02              # an input scalar; parity does not depend on its value


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def _bits(t):
    """device tensor -> numpy with BF16 as uint16 and E4M3 as uint8."""
    return host(t)


def _check_k_rows(k_in, pos, got, cfg, w, cache_dtype, k_scale):
    n, H, D = k_in.shape
    ref = np.zeros(((n + B - 1) // B, B, H, D), oracle.NP_TYPES[cache_dtype])
    oracle.cache_write_k(k_in, "bf16", np.arange(n, dtype=np.int64), ref, cache_dtype,
                         num_kv_heads=H, head_dim=D, block_size=B, norm_weight=w,
                         eps=cfg["eps"], pos_t=pos, theta=cfg["theta"], k_scale=k_scale,
                         nthreads=8)
    ref = ref.reshape(-1, H, D)[:n]
    st = {}
    ok = bf16_ok(got, ref, stats=st) if cache_dtype == "bf16" else e4m3_ok(got, ref)
    if st:
        say(f"  BF16 K: {st['n']} elements, {st['exact']} exact, {st['floor_only']} more than "
            f"1 ulp apart within the 2^-20 row floor")
    assert ok.all(), f"{int((~ok).sum())} K elements outside the bar"


def _check_v_rows(v_in, got_rows, v_kind, H, D):
    """v_in [n, H, D] BF16 bits; got_rows: [n, H, D] (copy / E4M3) or, for
    TQ, (codes [n, H, D], scale bytes [n, H, D/16]) in slot order."""
    n = v_in.shape[0]
    if v_kind == "bf16":
        assert (got_rows == v_in).all()
        return
    if v_kind == "fp8":
        ref = np.zeros(((n + B - 1) // B, B, H, D), np.uint8)
        oracle.cache_write_v(v_in, "bf16", np.arange(n, dtype=np.int64), ref, num_kv_heads=H,
                             head_dim_v=D, block_size=B, cache_dtype="fp8", v_scale=V_SCALE)
        assert (got_rows == ref.reshape(-1, H, D)[:n]).all()
        return
    st = tq_compare(got_rows[0], got_rows[1], v_in, "bf16", int(v_kind[2]), H, D)
    say(f"  TQ rows: {st}")


def _gather_rows(pool, slots, v_kind, H, D):
    """Rows at the given slots from a device pool (numpy, cache dtype)."""
    s = torch.from_numpy(np.asarray(slots, np.int64)).cuda()
    if v_kind is not None and v_kind.startswith("tq"):
        blocks = _bits(pool.index_select(0, s // B))
        local = np.arange(len(slots)) * B + np.asarray(slots, np.int64) % B
        return tq_rows_by_slot(blocks, local, int(v_kind[2]), H, D)
    flat = pool.view(-1, H, D)
    return _bits(flat.index_select(0, s))


def _sub_pool(lay, seqs, k_pool, v_pool):
    """The blocks of the sampled sequences, gathered from the device pools,
    and their block tables renumbered into that sub-pool."""
    nblk = (lay.seq_lens.astype(np.int64) + B - 1) // B
    ids = np.unique(np.concatenate([lay.block_tables[s, :nblk[s]] for s in seqs]))
    new = np.full(lay.num_blocks, -1, np.int64)
    new[ids] = np.arange(ids.size)
    bt = np.zeros((len(seqs), lay.block_tables.shape[1]), np.int32)
    for i, s in enumerate(seqs):
        bt[i, :nblk[s]] = new[lay.block_tables[s, :nblk[s]]]
    idx = torch.from_numpy(ids).cuda()
    return _bits(k_pool.index_select(0, idx)), _bits(v_pool.index_select(0, idx)), bt


def _sample_seqs(lens, k, seed):
    rng = np.random.default_rng(seed)
    pick = {int(np.argmin(lens)), int(np.argmax(lens))}
    pick |= set(int(x) for x in rng.choice(len(lens), size=k, replace=False))
    return sorted(pick)


@pytest.mark.parametrize("name", sorted(bench.WORKLOADS))
def test_full_size_decode_step_sampled(name):
    idx, v_kind, window, use_sinks = bench.WORKLOADS[name]
    tq = int(v_kind[2]) if v_kind.startswith("tq") else 0
    lay = W.layout(idx)
    cfg = lay.cfg
    S, Hq, Hkv, D = lay.num_seqs, cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"]
    fp8 = cfg["k_cache_dtype"] == "fp8"
    k_dt = "fp8" if fp8 else "bf16"
    v_scale = V_SCALE if v_kind == "fp8" else 1.0
    say(f"full-size decode step {name}: {S} seqs, {lay.total_tokens} tokens, "
        f"pool {lay.num_blocks} blocks")
    dev = torch.device("cuda")
    k_pool = torch.empty((lay.num_blocks, B, Hkv, D),
                         dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16, device=dev)
    if tq:
        v_pool = torch.empty((lay.num_blocks, pkv.v_block_bytes(tq + 1, B, Hkv, D)),
                             dtype=torch.uint8, device=dev)
    else:
        v_pool = torch.empty((lay.num_blocks, B, Hkv, D),
                             dtype=torch.float8_e4m3fn if v_kind == "fp8" else torch.bfloat16,
                             device=dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    w_np = W.norm_weight(idx)
    w = torch.from_numpy(w_np.view(np.int16)).to(dev).view(torch.bfloat16)

    # population write (history = positions 0 .. n-2)
    lens = lay.seq_lens.astype(np.int64)
    Th = int((lens - 1).sum())
    start_h, cu_h, pos_h = W.positions_history(lay)
    k_hist = W.device_normal(idx, W.S_K, (Th, Hkv, D), torch.bfloat16, dev, outliers=fp8)
    v_hist = W.device_normal(idx, W.S_V, (Th, Hkv, D), torch.bfloat16, dev)
    slots_h = torch.empty(Th, dtype=torch.int64, device=dev)
    pkv.fill_slots(slots_h, bt, _i32(start_h), _i32(cu_h), B)
    # the benchmark's k_scale: max |stored FP32 K| / 448 over the history
    k_scale = bench.history_k_scale(k_hist, _i32(pos_h), w, cfg) if fp8 else 1.0
    if fp8:
        say(f"  k_scale = {k_scale:.6g} (the benchmark's)")
    pkv.cache_write_k_fused(k_hist, slots_h, k_pool, norm_weight=w, eps=cfg["eps"],
                            pos_t=_i32(pos_h), theta=cfg["theta"], k_scale=k_scale)
    pkv.cache_write_v(v_hist, slots_h, v_pool, v_scale=v_scale, tq_bits=tq)

    # the decode step: new token at position n - 1 of every sequence
    k_new = W.device_normal(idx, W.S_KNEW, (S, Hkv, D), torch.bfloat16, dev, outliers=fp8)
    v_new = W.device_normal(idx, W.S_VNEW, (S, Hkv, D), torch.bfloat16, dev)
    q = W.device_normal(idx, W.S_Q, (S, Hq, D), torch.bfloat16, dev, outliers=fp8)
    tau, stride = 0.0, 0
    if name in bench.SPARSE_V:
        tau, stride, heavy_len = bench.SPARSE_V[name]
        n_heavy = bench.heavy_keys(k_pool, q, lay, stride, heavy_len)
        say(f"  sparse V: threshold {tau:g}, {n_heavy} heavy keys")
    start_d, cu_d, pos_d = W.positions_decode(lay)
    slots_d = torch.empty(S, dtype=torch.int64, device=dev)
    pkv.fill_slots(slots_d, bt, _i32(start_d), _i32(cu_d), B)
    pkv.cache_write_k_fused(k_new, slots_d, k_pool, norm_weight=w, eps=cfg["eps"],
                            pos_t=_i32(pos_d), theta=cfg["theta"], k_scale=k_scale)
    pkv.cache_write_v(v_new, slots_d, v_pool, v_scale=v_scale, tq_bits=tq)
    sinks = W.normal(idx, W.S_SINKS, (Hq,)) if use_sinks else None
    ws = torch.empty(max(16, pkv.decode_workspace_bytes(S, Hq, Hkv, D, lay.max_blocks_per_seq,
                                                        B, 0, window)),
                     dtype=torch.uint8, device=dev)
    out = pkv.paged_decode_attn(q, k_pool, v_pool, bt, seq_lens, scale=D ** -0.5,
                                k_scale=k_scale, v_scale=v_scale, sliding_window=window,
                                sinks=None if sinks is None else torch.from_numpy(sinks).to(dev),
                                workspace=ws, v_tq_bits=tq, sparse_v_threshold=tau)
    torch.cuda.synchronize()

    # slots of the step: all of them
    ref_slots = oracle.fill_slots(lay.block_tables, start_d, cu_d, S, B)
    assert (host(slots_d) == ref_slots).all()

    # K and V rows: sampled history tokens and the new tokens of every
    # sequence (with E4M3 K at the benchmark's k_scale, where a new token can
    # saturate)
    rng = np.random.default_rng(idx)
    hist_tok = np.sort(rng.choice(Th, size=96, replace=False))
    if stride:                                  # heavy keys were written over the K write's
        hist_tok = hist_tok[pos_h[hist_tok] % stride != 0]
    seqs = _sample_seqs(lens, 4, 100 + idx)
    tok_idx = torch.from_numpy(hist_tok).to(dev)
    h_slots = host(slots_h)[hist_tok]
    if fp8:
        new_codes = _gather_rows(k_pool, ref_slots, None, Hkv, D)
        say(f"  new tokens' K: {int(((new_codes & 0x7F) == 0x7E).sum())} of {new_codes.size} "
            f"codes saturated")
    for rows_k, rows_v, slots, pos in (
            (_bits(k_hist.index_select(0, tok_idx)), _bits(v_hist.index_select(0, tok_idx)),
             h_slots, pos_h[hist_tok]),
            (_bits(k_new), _bits(v_new), ref_slots, pos_d)):
        _check_k_rows(rows_k, pos, _gather_rows(k_pool, slots, None, Hkv, D), cfg, w_np,
                      k_dt, k_scale)
        _check_v_rows(rows_v, _gather_rows(v_pool, slots, v_kind, Hkv, D), v_kind, Hkv, D)

    # attention output of sampled sequences
    kp, vp, bt_sub = _sub_pool(lay, seqs, k_pool, v_pool)
    qs = _bits(q)[seqs]
    kw = dict(num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D, block_size=B,
              scale=D ** -0.5, k_scale=k_scale, v_scale=v_scale, sliding_window=window,
              sinks=sinks, nthreads=8)
    ref = oracle.paged_decode(qs, "bf16", kp, k_dt, vp, v_kind, bt_sub, lay.seq_lens[seqs], **kw)
    got = host(out)[seqs]
    if tau:
        # the skip leaves out a subset of the positions whose softmax weight
        # is at most tau: within the oracle's bound of its sparse output
        sp, bound = oracle.paged_decode_sparse_v(qs, "bf16", kp, k_dt, vp, v_kind, bt_sub,
                                                 lay.seq_lens[seqs], tau=tau, **kw)
        den = np.abs(ref).max(axis=-1, keepdims=True)
        err = float(((np.abs(got - sp) - bound) / np.where(den > 0, den, 1.0)).max())
        say(f"  sequences {seqs}: excess over the sparse-V bound {err:.3e}, "
            f"exact vs sparse {attn_err(ref, sp):.3e}")
    else:
        err = attn_err(got, ref)
    say(f"  sequences {seqs} (lengths {lens[seqs].tolist()}): err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


def test_full_size_prefill_sampled():
    name = "prefill_bf16_256seq_chunk256"
    idx, chunk = bench.PREFILL_WORKLOADS[name]
    lay = W.layout(idx)
    cfg = lay.cfg
    S, Hq, Hkv, D = lay.num_seqs, cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"]
    say(f"full-size prefill {name}: {S} seqs, chunk {chunk}")
    dev = torch.device("cuda")
    lens = lay.seq_lens.astype(np.int64)
    qlens = np.minimum(lens, chunk)
    Tc = int(qlens.sum())
    # the whole cache (history and chunk rows) written through the library
    start, cu, pos = W.positions_all(lay)
    T = int(cu[-1])
    k_pool = torch.empty((lay.num_blocks, B, Hkv, D), dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty_like(k_pool)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    w = torch.from_numpy(W.norm_weight(idx).view(np.int16)).to(dev).view(torch.bfloat16)
    k_all = W.device_normal(idx, W.S_K, (T, Hkv, D), torch.bfloat16, dev)
    v_all = W.device_normal(idx, W.S_V, (T, Hkv, D), torch.bfloat16, dev)
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    pkv.fill_slots(slots, bt, _i32(start), _i32(cu), B)
    pkv.cache_write_k_fused(k_all, slots, k_pool, norm_weight=w, eps=cfg["eps"], pos_t=_i32(pos),
                            theta=cfg["theta"])
    pkv.cache_write_v(v_all, slots, v_pool)
    del k_all, v_all
    cu_q = np.concatenate([[0], np.cumsum(qlens)]).astype(np.int32)
    q = W.device_normal(idx, W.S_Q, (Tc, Hq, D), torch.bfloat16, dev)
    out = pkv.paged_prefill_attn(q, _i32(cu_q), k_pool, v_pool, bt,
                                 torch.from_numpy(lay.seq_lens).to(dev), max_q_len=chunk,
                                 scale=D ** -0.5)
    torch.cuda.synchronize()
    seqs = _sample_seqs(lens, 1, 7)
    kp, vp, bt_sub = _sub_pool(lay, seqs, k_pool, v_pool)
    qh = _bits(q)
    qs = np.concatenate([qh[cu_q[s]:cu_q[s + 1]] for s in seqs])
    cu_sub = np.concatenate([[0], np.cumsum(qlens[seqs])]).astype(np.int32)
    ref = oracle.paged_prefill(qs, "bf16", cu_sub, kp, "bf16", vp, "bf16", bt_sub,
                               lay.seq_lens[seqs], num_q_heads=Hq, num_kv_heads=Hkv,
                               head_dim_qk=D, head_dim_v=D, block_size=B, scale=D ** -0.5,
                               nthreads=8)
    oh = host(out)
    got = np.concatenate([oh[cu_q[s]:cu_q[s + 1]] for s in seqs])
    err = attn_err(got, ref)
    say(f"  sequences {seqs} (lengths {lens[seqs].tolist()}): err {err:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL


@pytest.mark.parametrize("v_kind", ["bf16", "tq3"])
def test_pool_beyond_4gib(v_kind):
    """Sequences whose blocks lie past 4 GiB of a 5.8 GiB pool (BF16 K; BF16
    or TQ3 V): slot fill, K and V writes, and decode reach them through
    64-bit offsets."""
    Hq, Hkv, D = 32, 8, 128
    nb = 180_000                                  # x 32 KiB per BF16 block = 5.5 GiB
    lens = np.array([1, 700, 2500, 5000], np.int32)
    nblk = (lens + B - 1) // B
    M = int(nblk.max())
    # each sequence's blocks: the last ones of the pool, shuffled
    rng = np.random.default_rng(11)
    top = rng.permutation(np.arange(nb - int(nblk.sum()), nb)).astype(np.int32)
    bt = np.zeros((lens.size, M), np.int32)
    off = 0
    for s, k in enumerate(nblk):
        bt[s, :k] = top[off:off + k]
        off += k
    lay = W.Layout(2, lens, bt, nb, -1, B)
    assert int(bt.max()) * B * Hkv * D * 2 >= 1 << 32
    tq = 3 if v_kind == "tq3" else 0
    say(f"pool of {nb} blocks, V {v_kind}: blocks {int(bt[bt > 0].min())}..{int(bt.max())}")
    dev = torch.device("cuda")
    k_pool = torch.zeros((nb, B, Hkv, D), dtype=torch.bfloat16, device=dev)
    if tq:
        v_pool = torch.zeros((nb, pkv.v_block_bytes(tq + 1, B, Hkv, D)), dtype=torch.uint8,
                             device=dev)
    else:
        v_pool = torch.zeros_like(k_pool)
    cfg = W.WORKLOADS[2]
    start, cu, pos = W.positions_all(lay)
    T = int(cu[-1])
    k_in = W.device_normal(2, 501, (T, Hkv, D), torch.bfloat16, dev)
    v_in = W.device_normal(2, 502, (T, Hkv, D), torch.bfloat16, dev)
    w_np = W.norm_weight(2)
    w = torch.from_numpy(w_np.view(np.int16)).to(dev).view(torch.bfloat16)
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    bt_d = torch.from_numpy(bt).to(dev)
    pkv.fill_slots(slots, bt_d, _i32(start), _i32(cu), B)
    pkv.cache_write_k_fused(k_in, slots, k_pool, norm_weight=w, eps=cfg["eps"], pos_t=_i32(pos),
                            theta=cfg["theta"])
    pkv.cache_write_v(v_in, slots, v_pool, tq_bits=tq)
    q = W.device_normal(2, 503, (lens.size, Hq, D), torch.bfloat16, dev)
    out = pkv.paged_decode_attn(q, k_pool, v_pool, bt_d, torch.from_numpy(lens).to(dev),
                                scale=D ** -0.5, v_tq_bits=tq)
    torch.cuda.synchronize()
    ref_slots = oracle.fill_slots(bt, start, cu, T, B)
    assert (host(slots) == ref_slots).all() and ref_slots.max() * Hkv * D * 2 >= 1 << 32
    pick = np.sort(rng.choice(T, size=64, replace=False))
    idx = torch.from_numpy(pick).to(dev)
    _check_k_rows(_bits(k_in.index_select(0, idx)), pos[pick],
                  _gather_rows(k_pool, ref_slots[pick], None, Hkv, D), cfg, w_np, "bf16", 1.0)
    _check_v_rows(_bits(v_in.index_select(0, idx)),
                  _gather_rows(v_pool, ref_slots[pick], v_kind, Hkv, D), v_kind, Hkv, D)
    seqs = list(range(lens.size))
    kp, vp, bt_sub = _sub_pool(lay, seqs, k_pool, v_pool)
    ref = oracle.paged_decode(_bits(q), "bf16", kp, "bf16", vp, v_kind, bt_sub, lens,
                              num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D,
                              block_size=B, scale=D ** -0.5, nthreads=8)
    err = attn_err(host(out), ref)
    say(f"  err {err:.3e}")
    assert np.isfinite(host(out)).all() and err <= ATTN_TOL
