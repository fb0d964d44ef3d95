"""GPU parity of the slot mapping, the fused K write and the V write against
the CPU oracle, through the C ABI (via the package binding).

Slots and V: bit-exact over the whole output.  K: every byte of the pool is
compared -- written rows within the K bar, every other byte unchanged from a
sentinel fill."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import bf16_ok, dev, e4m3_ok, f32_ok, host, say

pytestmark = pytest.mark.gpu


def gpu_slots(lay, start, cu):
    T = int(cu[-1])
    slots = torch.empty(T, dtype=torch.int64, device="cuda")
    pkv.fill_slots(slots, dev(lay.block_tables), dev(start.astype(np.int32)),
                   dev(cu.astype(np.int32)), lay.block_size)
    return slots


# ---------------------------------------------------------------- slots

@pytest.mark.parametrize("index,nseq", [(0, None), (1, None), (2, 64), (3, 8)])
def test_fill_slots_bit_exact(index, nseq):
    lay = W.layout(index, num_seqs=nseq)
    for name, fn in (("all", W.positions_all), ("decode", W.positions_decode)):
        start, cu, _ = fn(lay)
        say(f"fill_slots workload {index} {name}: {int(cu[-1])} tokens")
        got = host(gpu_slots(lay, start, cu))
        ref = oracle.fill_slots(lay.block_tables, start, cu, int(cu[-1]), lay.block_size)
        assert (got == ref).all()


def test_fill_slots_edge_cases():
    """Negative table entries, positions past the table, uncovered tokens."""
    bt = np.array([[5, 2, 9], [7, 0, 3], [-1, 4, 1], [6, 8, 11]], np.int32)
    start = np.array([0, 6, 2, 10], np.int32)
    counts = np.array([10, 3, 6, 3])
    cu = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(cu[-1]) + 5                          # 5 tokens no sequence covers
    slots = torch.full((T,), 123, dtype=torch.int64, device="cuda")
    pkv.fill_slots(slots, dev(bt), dev(start), dev(cu), 4)
    ref = oracle.fill_slots(bt, start, cu, T, 4)
    got = host(slots)
    assert (got == ref).all()
    assert (got[-5:] == -1).all() and got[int(cu[-1]) - 1] == -1


# ---------------------------------------------------------------- V

def test_v_write_bit_exact_whole_pool():
    lay = W.layout(1)
    start, cu, _ = W.positions_all(lay)
    T = int(cu[-1])
    slots_np = oracle.fill_slots(lay.block_tables, start, cu, T, 16)
    slots_np[::97] = -1                          # padding tokens
    v = W.kv_tokens(1, T, "v")
    ref = np.full((lay.num_blocks, 16, 8, 128), 0xBEEF, np.uint16)
    oracle.cache_write_v(v, "bf16", slots_np, ref, num_kv_heads=8, head_dim_v=128, block_size=16)
    pool = dev(np.full_like(ref, 0xBEEF))
    say(f"cache_write_v workload 1: {T} tokens")
    pkv.cache_write_v(dev(v), dev(slots_np), pool)
    assert (host(pool) == ref).all()


def test_v_write_f32_strided_and_out_of_pool_slots():
    T, H, D = 37, 64, 128
    stride_rows = W.normal(4, 120, (T, H * D + 64))
    v = torch.from_numpy(stride_rows).cuda()[:, :H * D].view(T, H, D)
    nb = 4
    slots_np = np.arange(T, dtype=np.int64) * 3 % (nb * 16)
    slots_np[[2, 5, 9]] = [-7, nb * 16, nb * 16 + 100]     # skipped
    ref = np.full((nb, 16, H, D), -3.5, np.float32)
    oracle.cache_write_v(stride_rows, "f32", slots_np, ref, num_kv_heads=H, head_dim_v=D,
                         block_size=16, in_token_stride=H * D + 64)
    pool = dev(np.full_like(ref, -3.5))
    pkv.cache_write_v(v, dev(slots_np), pool)
    assert host(pool).tobytes() == ref.tobytes()


# ---------------------------------------------------------------- K

def k_case(index, T, cache_dtype, *, pos=None, mrope=False, nope=False, norm=True,
           k_scale=1.0, lay=None):
    cfg = W.WORKLOADS[index]
    H, D, B = cfg["num_kv_heads"], cfg["head_dim"], cfg["block_size"]
    R, off, theta, eps = cfg["rotary_dim"], cfg["rope_offset"], cfg["theta"], cfg["eps"]
    in_dt = cfg["kv_dtype"]
    k = W.kv_tokens(index, T, "k")
    w = W.norm_weight(index) if norm else None
    if lay is None:
        nb = (T + B - 1) // B + 3
        slots_np = np.random.default_rng(index).permutation(nb * B)[:T].astype(np.int64)
    else:
        nb = lay.num_blocks
        start, cu, _ = W.positions_all(lay)
        slots_np = oracle.fill_slots(lay.block_tables, start, cu, T, B)
    pos = np.arange(T, dtype=np.int32) if pos is None else pos
    sentinel = {"bf16": 0x7FA1, "fp8": 0x5A, "f32": np.float32(-7.25)}[cache_dtype]
    ref = np.full((nb, B, H, D), sentinel, oracle.NP_TYPES[cache_dtype])
    ph = pos if mrope else None
    oracle.cache_write_k(k, in_dt, slots_np, ref, cache_dtype, num_kv_heads=H, head_dim=D,
                         block_size=B, norm_weight=w, eps=eps, pos_t=pos, pos_h=ph, pos_w=ph,
                         theta=theta, rope_offset=off, rotary_dim=R, nope=nope, k_scale=k_scale,
                         nthreads=8)
    gref = dev(ref) if cache_dtype != "f32" else torch.from_numpy(ref.copy()).cuda()
    pt = dev(pos)
    say(f"cache_write_k workload {index}: {T} tokens -> {cache_dtype} mrope={mrope} nope={nope}")
    pkv.cache_write_k_fused(dev(k), dev(slots_np), gref, norm_weight=None if w is None else dev(w),
                            eps=eps, pos_t=pt, pos_h=pt if mrope else None,
                            pos_w=pt if mrope else None, theta=theta, rope_offset=off,
                            rotary_dim=R, nope=nope, k_scale=k_scale)
    got = host(gref)
    return got, ref, slots_np


def check_k(got, ref, slots_np, cache_dtype, sentinel_check=True):
    H, D = got.shape[2], got.shape[3]
    rows_g = got.reshape(-1, H, D)
    rows_r = ref.reshape(-1, H, D)
    written = np.zeros(rows_g.shape[0], bool)
    valid = slots_np[(slots_np >= 0) & (slots_np < rows_g.shape[0])]
    written[valid] = True
    if sentinel_check:
        assert rows_g[~written].tobytes() == rows_r[~written].tobytes(), "rows outside the slots changed"
    g, r = rows_g[written], rows_r[written]
    if cache_dtype == "bf16":
        st = {}
        ok = bf16_ok(g, r, stats=st)
        exact = float((g == r).mean())
        say(f"  BF16 K: {st['n']} elements, {st['floor_only']} more than 1 ulp apart within "
            f"the 2^-20 row floor")
    elif cache_dtype == "fp8":
        ok = e4m3_ok(g, r)
        exact = float((g == r).mean())
    else:
        ok = f32_ok(g, r)
        exact = float((g == r).mean())
    say(f"  exact-match fraction {exact:.5f}, failures {int((~ok).sum())}")
    assert ok.all()
    return exact


def test_k_write_tiny_workload():
    lay = W.layout(0)
    got, ref, s = k_case(0, lay.total_tokens, "bf16", lay=lay)
    check_k(got, ref, s, "bf16")


def test_k_write_prefill_bf16_and_mrope_bit_identical():
    lay = W.layout(1)
    T = lay.total_tokens
    _, _, pos = W.positions_all(lay)
    got, ref, s = k_case(1, T, "bf16", pos=pos, lay=lay)
    exact = check_k(got, ref, s, "bf16")
    assert exact > 0.99
    got_m, ref_m, _ = k_case(1, T, "bf16", pos=pos, mrope=True, lay=lay)
    assert got_m.tobytes() == got.tobytes(), "MRoPE with equal positions differs from scalar"
    assert ref_m.tobytes() == ref.tobytes()


def test_k_write_mrope_distinct_positions():
    T = 300
    cfg = W.WORKLOADS[1]
    k = W.kv_tokens(1, T, "k")
    w = W.norm_weight(1)
    pt = (np.arange(T) * 3).astype(np.int32)
    ph = (np.arange(T) * 5 + 100).astype(np.int32)
    pw = (np.arange(T) * 7 + 9).astype(np.int32)
    slots_np = np.arange(T, dtype=np.int64)
    nb = (T + 15) // 16
    ref = np.zeros((nb, 16, 8, 128), np.uint16)
    oracle.cache_write_k(k, "bf16", slots_np, ref, "bf16", num_kv_heads=8, head_dim=128,
                         block_size=16, norm_weight=w, pos_t=pt, pos_h=ph, pos_w=pw)
    g = dev(np.zeros_like(ref))
    pkv.cache_write_k_fused(dev(k), dev(slots_np), g, norm_weight=dev(w), pos_t=dev(pt),
                            pos_h=dev(ph), pos_w=dev(pw), theta=cfg["theta"])
    check_k(host(g), ref, slots_np, "bf16")


def test_k_write_fp8_long_positions():
    """FP8 store at decode-length positions (up to 32767) with saturation."""
    T = 2048
    pos = np.random.default_rng(3).integers(0, 32768, T).astype(np.int32)
    # scale chosen so that the largest values saturate
    got, ref, s = k_case(3, T, "fp8", pos=pos, k_scale=0.02)
    check_k(got, ref, s, "fp8")
    assert (got == 0x7E).any() or (got == 0xFE).any()


def test_k_write_fp8_and_f32_stores_bf16_input():
    T = 777
    pos = (np.arange(T) * 41).astype(np.int32)
    for cdt, ks in (("fp8", 0.0125), ("f32", 1.0)):
        got, ref, s = k_case(2, T, cdt, pos=pos, k_scale=ks)
        check_k(got, ref, s, cdt)


def test_k_write_mla_style_f32_partial_rope_and_nope():
    """D 192 = 128 NoPE + 64 rotated dims at offset 128, theta 5e4, FP32 in and
    out, no norm; and the NoPE flag (no rotation at all)."""
    T = 64
    pos = np.arange(4032, 4032 + T, dtype=np.int32)
    for nope in (False, True):
        got, ref, s = k_case(4, T, "f32", pos=pos, nope=nope, norm=False)
        check_k(got, ref, s, "f32")


def test_k_write_head_dims_and_partial_rotary():
    """Other supported layouts: D 64/128/256, partial rotary, FP32 input.  The
    E4M3 store's lane exchange runs with 4, 8 and 16 lanes per row, 2, 4, 6 and
    8 chunks per lane, and one lane per row (rotary_dim 48: an odd pair
    distance in chunks)."""
    rng = np.random.default_rng(11)
    for (in_dt, D, R, off, H) in (("bf16", 64, 64, 0, 4), ("bf16", 128, 64, 0, 2),
                                  ("bf16", 256, 256, 0, 2), ("f32", 128, 128, 0, 2),
                                  ("f32", 64, 32, 32, 8), ("bf16", 192, 64, 128, 3),
                                  ("bf16", 64, 48, 0, 2)):
        T = 50
        x = rng.standard_normal((T, H, D)).astype(np.float32)
        k = W.bf16_bits(x) if in_dt == "bf16" else x
        wv = rng.uniform(0.5, 1.5, D).astype(np.float32)
        w = W.bf16_bits(wv) if in_dt == "bf16" else wv
        pos = rng.integers(0, 20000, T).astype(np.int32)
        slots_np = rng.permutation(64)[:T].astype(np.int64)
        for cdt in ("bf16", "fp8"):
            ref = np.zeros((4, 16, H, D), oracle.NP_TYPES[cdt])
            oracle.cache_write_k(k, in_dt, slots_np, ref, cdt, num_kv_heads=H, head_dim=D,
                                 block_size=16, norm_weight=w, pos_t=pos, theta=10000.0,
                                 rope_offset=off, rotary_dim=R, k_scale=0.03)
            g = dev(np.zeros_like(ref))
            say(f"K layout {in_dt} D={D} R={R} off={off} H={H} -> {cdt}")
            pkv.cache_write_k_fused(dev(k), dev(slots_np), g, norm_weight=dev(w), pos_t=dev(pos),
                                    theta=10000.0, rope_offset=off, rotary_dim=R, k_scale=0.03)
            check_k(host(g), ref, slots_np, cdt)


@pytest.mark.parametrize("T,H,D", [(140_003, 3, 128), (140_003, 5, 64), (24_581, 3, 128)])
def test_k_write_fp8_many_units_per_wave(T, H, D):
    """E4M3 stores from BF16 rows with enough tokens that a wave takes several
    (token, head-group) units (16 for the first two cases, 3 for the last:
    the rows of the next two units are in flight while one is stored), with
    an odd head count (rows past the last head in every unit), 1% padding
    slots and a last wave with fewer units; the whole pool is compared."""
    rng = np.random.default_rng(T + H)
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    k = W.bf16_bits(x)
    w = W.bf16_bits(rng.uniform(0.5, 1.5, D).astype(np.float32))
    nb = (int(T * 1.02) + 15) // 16
    slots_np = rng.permutation(nb * 16)[:T].astype(np.int64)
    slots_np[rng.random(T) < 0.01] = -1
    pos = rng.integers(0, 32768, T).astype(np.int32)
    ref = np.full((nb, 16, H, D), 0x5A, np.uint8)
    oracle.cache_write_k(k, "bf16", slots_np, ref, "fp8", num_kv_heads=H, head_dim=D,
                         block_size=16, norm_weight=w, pos_t=pos, theta=10000.0, rotary_dim=D,
                         k_scale=0.01, nthreads=16)
    g = dev(np.full_like(ref, 0x5A))
    say(f"E4M3 K write, {T} tokens, H={H}, D={D}")
    pkv.cache_write_k_fused(dev(k), dev(slots_np), g, norm_weight=dev(w), pos_t=dev(pos),
                            theta=10000.0, rotary_dim=D, k_scale=0.01)
    got = host(g)
    check_k(got, ref, slots_np, "fp8")
    assert (got == 0x7E).any() or (got == 0xFE).any()     # some rows saturate


def _stratified_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x1234, 0xC000], np.uint32)
    return (hi[:, None] | lows[None, :]).reshape(-1)


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_store_rounding_matches_oracle_on_all_exponents(cache_dtype):
    """No norm, no rotation, FP32 input, k_scale 1: the K write is the bare
    rounding, so the codes must equal the oracle's exactly for every sign,
    exponent and upper mantissa pattern (NaN: both NaN)."""
    pat = _stratified_patterns()
    x = pat.view(np.float32).reshape(-1, 1, 64)
    T = x.shape[0]
    slots_np = np.arange(T, dtype=np.int64)
    nb = T // 16
    ref = np.zeros((nb, 16, 1, 64), oracle.NP_TYPES[cache_dtype])
    oracle.cache_write_k(x, "f32", slots_np, ref, cache_dtype, num_kv_heads=1, head_dim=64,
                         block_size=16, nope=True, k_scale=1.0, nthreads=8)
    g = dev(np.zeros_like(ref))
    say(f"rounding sweep -> {cache_dtype}: {x.size} values")
    pkv.cache_write_k_fused(torch.from_numpy(x).cuda(), dev(slots_np), g, nope=True, k_scale=1.0)
    got = host(g).reshape(-1)
    r = ref.reshape(-1)
    if cache_dtype == "bf16":
        gn = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
        rn = ((r & 0x7F80) == 0x7F80) & ((r & 0x7F) != 0)
    else:
        gn = (got & 0x7F) == 0x7F
        rn = (r & 0x7F) == 0x7F
    bad = np.nonzero(((got != r) & ~rn) | (gn != rn))[0]
    if bad.size:
        xs = x.reshape(-1)[bad[:8]]
        say(f"  {bad.size} mismatches; first (input bits, gpu, oracle):",
            [(hex(int(v.view(np.uint32))), hex(int(a)), hex(int(b)))
             for v, a, b in zip(xs, got[bad[:8]], r[bad[:8]])])
    assert (gn == rn).all(), "NaN placement differs"
    assert bad.size == 0
