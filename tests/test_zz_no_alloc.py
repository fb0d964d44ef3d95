"""The no-allocation decode entry point, pkv_paged_decode_attn_noalloc, called
through the C ABI: its output against pkv_paged_decode_attn's on the same
inputs (the same kernels and plan, so bit for bit), on two calls in a row,
the second with a smaller input (the library's scratch keeps the first
call's partials, which the second must not read), for the balanced plan
(BF16 and E4M3-K caches), the split plan (sliding window) and the FP32 path
(query rotation, gate).  The small calls are also held to the oracle (2e-3)."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, host, say

pytestmark = pytest.mark.gpu
B = 16


def _pools(idx, nb, H, D, k_fp8, dev):
    k = W.device_normal(idx, 901, (nb, B, H, D), torch.bfloat16, dev)
    if k_fp8:
        k = (k.float() * 4).clamp(-448, 448).to(torch.float8_e4m3fn)
    v = W.device_normal(idx, 902, (nb, B, H, D), torch.bfloat16, dev)
    return k, v


def _both(q, kp, vp, lay, dev, **kw):
    bt = torch.from_numpy(lay.block_tables).to(dev)
    sl = torch.from_numpy(lay.seq_lens).to(dev)
    ref = pkv.paged_decode_attn(q, kp, vp, bt, sl, **kw)
    out = torch.full_like(ref, float("nan"))
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    pkv.paged_decode_attn_noalloc(q, kp, vp, bt, sl, out=out, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return out, ref


@pytest.mark.parametrize("k_fp8", [False, True])
@pytest.mark.parametrize("window", [0, 1000])
def test_noalloc_decode_matches_the_workspace_call(k_fp8, window):
    dev = torch.device("cuda")
    Hq, H, D = 32, 8, 128
    big = W.layout(2, num_seqs=40)                       # U[512, 8192] lengths
    lens_small = np.array([1, 17, 300, 2048, 5], np.int32)
    nb = big.num_blocks
    kp, vp = _pools(2, nb, H, D, k_fp8, dev)
    # the small call's tables: blocks of the same pool
    small = W.Layout(2, lens_small, big.block_tables[:5, :128].copy(), nb, big.pad_block, B)
    kw = dict(scale=D ** -0.5, k_scale=0.5 if k_fp8 else 1.0, sliding_window=window)
    for lay in (big, small):
        need = pkv.decode_workspace_bytes(lay.num_seqs, Hq, H, D, lay.max_blocks_per_seq, B, 0,
                                          window)
        say(f"noalloc decode: S={lay.num_seqs} tokens={lay.total_tokens} fp8K={k_fp8} "
            f"window={window} partials={need} B")
        q = W.device_normal(2, 903 + lay.num_seqs, (lay.num_seqs, Hq, D), torch.bfloat16, dev)
        out, ref = _both(q, kp, vp, lay, dev, **kw)
        assert torch.equal(out, ref), "noalloc output differs from the workspace call's"
    # the small call against the oracle, over the blocks it reads
    ids = np.unique(small.block_tables)
    remap = np.full(nb, -1, np.int64)
    remap[ids] = np.arange(ids.size)
    idx = torch.from_numpy(ids.astype(np.int64)).to(dev)
    kh = host(kp.index_select(0, idx))
    vh = host(vp.index_select(0, idx))
    want = oracle.paged_decode(host(q), "bf16", kh, "fp8" if k_fp8 else "bf16", vh, "bf16",
                               remap[small.block_tables].astype(np.int32), lens_small,
                               num_q_heads=Hq, num_kv_heads=H, head_dim_qk=D, head_dim_v=D,
                               block_size=B, scale=D ** -0.5, k_scale=kw["k_scale"],
                               sliding_window=window, nthreads=8)
    err = attn_err(host(out), want)
    say(f"  small call vs oracle: {err:.3e}")
    assert np.isfinite(host(out)).all() and err <= ATTN_TOL


def test_noalloc_decode_fp32_path_rotation_and_gate():
    dev = torch.device("cuda")
    H, Dqk, Dv = 64, 192, 128
    n_big, n_small = 4096, 700
    nb = n_big // B
    kp = W.device_normal(4, 911, (nb, B, H, Dqk), torch.float32, dev)
    vp = W.device_normal(4, 912, (nb, B, H, Dv), torch.float32, dev)
    bt = np.arange(nb, dtype=np.int32).reshape(1, -1)
    kw = dict(scale=Dqk ** -0.5, q_rope=True, q_rope_theta=5e4, q_rope_offset=128,
              q_rope_dim=64)
    for n in (n_big, n_small):
        lay = W.Layout(4, np.array([n], np.int32), bt, nb, -1, B)
        q = W.device_normal(4, 913 + n, (1, H, Dqk), torch.float32, dev)
        gate = torch.rand((1, H, Dv), generator=torch.Generator(device=dev).manual_seed(n),
                          device=dev)
        say(f"noalloc FP32 decode: n={n}, partials="
            f"{pkv.decode_workspace_bytes(1, H, H, Dv, nb, B)} B")
        out, ref = _both(q, kp, vp, lay, dev, gate=gate, **kw)
        assert torch.equal(out, ref), "noalloc output differs from the workspace call's"
    want = oracle.paged_decode(host(q), "f32", host(kp), "f32", host(vp), "f32", bt,
                               np.array([n_small], np.int32), num_q_heads=H, num_kv_heads=H,
                               head_dim_qk=Dqk, head_dim_v=Dv, block_size=B, gate=host(gate),
                               nthreads=8, **kw)
    err = attn_err(host(out), want)
    say(f"  small call vs oracle: {err:.3e}")
    assert err <= ATTN_TOL


def test_noalloc_rejects_partials_beyond_the_scratch():
    dev = torch.device("cuda")
    S, Hq, H, D, M = 1024, 64, 8, 128, 4096
    q = torch.zeros((S, Hq, D), dtype=torch.bfloat16, device=dev)
    kp = torch.zeros((2, B, H, D), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((S, M), dtype=torch.int32, device=dev)
    sl = torch.ones(S, dtype=torch.int32, device=dev)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    with pytest.raises(pkv.PkvError) as e:
        pkv.paged_decode_attn_noalloc(q, kp, kp, bt, sl, out=out, scale=0.1)
    assert e.value.status == -3 and "scratch" in str(e.value)
