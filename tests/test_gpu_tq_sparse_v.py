"""GPU parity of the sparse-V skip of the TQ V decode (sparse_v_threshold)
against the oracle's sparse-V decode.

The kernel leaves out a position when exp(s_t - running max) <= tau; the
oracle defines the output over the positions whose softmax weight exceeds
tau.  The first is a subset test of the second, so in general the kernel
lies within the oracle's ``bound`` of its ``out``.  Where the inputs fix the
kernel's choice, the two agree at the attention bar (2e-3 row-relative):

* every 16-token block holds a dominant position (and the first position
  of a sliding window is one), whose score exceeds every other score of the
  block by 5.5-6.2, while the dominant scores of a query head lie within
  0.15 of each other: then in any piece of any split plan each other
  position has exp(s - running max) <= 4e-3 < tau = 1e-2 and each dominant
  one >= 0.86, and the softmax weights are <= 4e-3 and >= 0.014 (at most 63
  dominant positions): both leave out exactly the non-dominant positions;
* one dominant position at the start of a sequence read as one piece
  (split_tokens 2048): every later position has exp(s - s_0) <= 4e-3, so
  every later block is skipped whole by the kernel, and left out by the
  oracle (weights <= 4e-3 against >= 0.12).
These margins were computed from the same seeded inputs in FP64.

The other positions' V rows are four times larger, so that leaving them out
moves the output by far more than the bar (checked against the exact decode).
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import ATTN_TOL, attn_err, dev, host, say

pytestmark = pytest.mark.gpu

D = 128
TAU = 1e-2


def _slots(lay, s, toks):
    bt = lay.block_tables[s]
    return np.array([bt[t // 16] * 16 + t % 16 for t in toks], np.int64)


def _peaked(lay, Hkv, G, bits, k_dt, seed, dominant):
    """q, K pool and TQ V pool: K rows of dominant positions (the
    `dominant(s, n)` token lists) carry 8 in dimension 0, others 0; query head
    h has 8 + 0.25 (h % 4) there; dimensions 1.. are noise.  V rows of the
    other positions are four times larger."""
    Hq = Hkv * G
    nb = lay.num_blocks
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((lay.num_seqs, Hq, D)).astype(np.float32)
    q[:, :, 0] = 8.0 + 0.25 * (np.arange(Hq) % 4)
    k = (rng.standard_normal((nb * 16, Hkv, D)) * 0.02).astype(np.float32)
    k[:, :, 0] = 0.0
    big = np.ones(nb * 16, bool)
    for s in range(lay.num_seqs):
        n = int(lay.seq_lens[s])
        sl = _slots(lay, s, dominant(s, n))
        k[sl, :, 0] = 8.0
        big[sl] = False
    x = rng.standard_normal((nb * 16, Hkv, D)).astype(np.float32)
    x[big] *= 4.0
    vp = np.zeros((nb, oracle.tq_block_bytes(bits, 16, Hkv, D)), np.uint8)
    oracle.cache_write_v(x, "f32", np.arange(nb * 16, dtype=np.int64), vp, num_kv_heads=Hkv,
                         head_dim_v=D, block_size=16, cache_dtype=f"tq{bits}")
    k = k.reshape(nb, 16, Hkv, D)
    kp = oracle.e4m3_from_f32(k / 0.5) if k_dt == "fp8" else W.bf16_bits(k)
    return W.bf16_bits(q), kp, vp


def _run(q, kp, k_dt, vp, bits, lay, Hq, Hkv, tau, *, window=0, sinks=None, split=0):
    kw = dict(num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=D, block_size=16,
              scale=D ** -0.5, k_scale=0.5 if k_dt == "fp8" else 1.0, sliding_window=window,
              sinks=sinks, nthreads=8)
    out, bound = oracle.paged_decode_sparse_v(q, "bf16", kp, k_dt, vp, f"tq{bits}",
                                              lay.block_tables, lay.seq_lens, tau=tau, **kw)
    ref = oracle.paged_decode(q, "bf16", kp, k_dt, vp, f"tq{bits}", lay.block_tables,
                              lay.seq_lens, **kw)
    say(f"sparse-V decode TQ{bits}: S={lay.num_seqs} tokens={lay.total_tokens} Hq={Hq} "
        f"Hkv={Hkv} K={k_dt} tau={tau} window={window} sinks={sinks is not None} split={split}")
    got = pkv.paged_decode_attn(dev(q), dev(kp), dev(vp, torch.uint8), dev(lay.block_tables),
                                dev(lay.seq_lens), scale=D ** -0.5, k_scale=kw["k_scale"],
                                sliding_window=window,
                                sinks=None if sinks is None else dev(sinks), split_tokens=split,
                                v_tq_bits=bits, sparse_v_threshold=tau)
    return host(got), out, bound, ref


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("k_dt", ["bf16", "fp8"])
@pytest.mark.parametrize("G", [1, 4, 16])
def test_one_dominant_position_per_block(bits, k_dt, G):
    lay = W.layout_for(2, [0, 1, 15, 16, 17, 300, 999, 640])
    Hkv = 2
    q, kp, vp = _peaked(lay, Hkv, G, bits, k_dt, 40 + bits,
                        lambda s, n: list(range(0, n, 16)))
    for split in (0, 16, 64):                # balanced ranges, one-block and four-block pieces
        got, out, bound, ref = _run(q, kp, k_dt, vp, bits, lay, Hkv * G, Hkv, TAU, split=split)
        err, moved = attn_err(got, out), attn_err(ref, out)
        say(f"  err vs sparse oracle {err:.3e}; exact vs sparse {moved:.3e}")
        assert np.isfinite(got).all() and (got[0] == 0).all()
        assert err <= ATTN_TOL and moved > 10 * ATTN_TOL


@pytest.mark.parametrize("bits", [3, 4])
def test_window_and_sinks(bits):
    lay = W.layout_for(2, [1, 17, 300, 999])
    Hkv, G, window = 2, 4, 100
    lo = lambda n: max(n - window, 0)
    q, kp, vp = _peaked(lay, Hkv, G, bits, "bf16", 60 + bits,
                        lambda s, n: sorted({lo(n)} | set(range(16 * (lo(n) // 16 + 1), n, 16))))
    sinks = np.full(Hkv * G, 5.0, np.float32)
    for split in (0, 32):
        got, out, bound, ref = _run(q, kp, "bf16", vp, bits, lay, Hkv * G, Hkv, TAU,
                                    window=window, sinks=sinks, split=split)
        err, moved = attn_err(got, out), attn_err(ref, out)
        say(f"  err vs sparse oracle {err:.3e}; exact vs sparse {moved:.3e}")
        assert np.isfinite(got).all() and err <= ATTN_TOL and moved > 10 * ATTN_TOL


@pytest.mark.parametrize("G", [1, 8])
def test_whole_blocks_skipped_after_a_dominant_first_position(G):
    """One piece per sequence, read in order: the first position sets the
    running maximum, every later block has no position kept."""
    lay = W.layout_for(2, [33, 700, 2048, 1999])
    Hkv = 2
    q, kp, vp = _peaked(lay, Hkv, G, 3, "bf16", 70 + G, lambda s, n: [0])
    got, out, bound, ref = _run(q, kp, "bf16", vp, 3, lay, Hkv * G, Hkv, TAU, split=2048)
    err, moved = attn_err(got, out), attn_err(ref, out)
    say(f"  err vs sparse oracle {err:.3e}; exact vs sparse {moved:.3e}")
    assert np.isfinite(got).all() and err <= ATTN_TOL and moved > 0.1


@pytest.mark.parametrize("split,Hkv", [(0, 4), (48, 4), (0, 3)])
def test_random_scores_within_the_bound(split, Hkv):
    """Unstructured peaked scores: the kernel's result lies within the
    oracle's bound of its sparse output (plus the attention bar); an odd
    kv-head count puts one kv head in each work-group."""
    lay = W.layout_for(3, [5, 100, 513, 4000, 2222])
    G = 4
    rng = np.random.default_rng(91)
    q = W.bf16_bits(rng.standard_normal((lay.num_seqs, Hkv * G, D)).astype(np.float32) * 3.0)
    kp = W.bf16_bits(rng.standard_normal((lay.num_blocks, 16, Hkv, D)).astype(np.float32))
    x = rng.standard_normal((lay.num_blocks * 16, Hkv, D)).astype(np.float32)
    vp = np.zeros((lay.num_blocks, oracle.tq_block_bytes(3, 16, Hkv, D)), np.uint8)
    oracle.cache_write_v(x, "f32", np.arange(lay.num_blocks * 16, dtype=np.int64), vp,
                         num_kv_heads=Hkv, head_dim_v=D, block_size=16, cache_dtype="tq3")
    for tau in (1e-4, 1e-3):
        got, out, bound, ref = _run(q, kp, "bf16", vp, 3, lay, Hkv * G, Hkv, tau, split=split)
        den = np.abs(ref).max(axis=-1, keepdims=True)
        excess = (np.abs(got - out) - bound) / np.where(den > 0, den, 1.0)
        say(f"  tau {tau}: max excess over the bound {excess.max():.3e}; "
            f"bound/row max {(bound / np.where(den > 0, den, 1.0)).max():.3e}")
        assert np.isfinite(got).all() and excess.max() <= ATTN_TOL
        assert (bound > 0).any()


def test_tiny_threshold_equals_the_exact_decode():
    """A threshold below every weight runs the skipping kernels and leaves
    nothing out: the exact call's output up to rounding (the skipping kernels
    rescale a pending block's weights instead of the accumulator, so their
    FP16 weights round differently: 1e-5 row-relative)."""
    lay = W.layout_for(2, [0, 1, 17, 300, 999])
    Hkv, G, bits = 2, 4, 3
    q, kp, vp = _peaked(lay, Hkv, G, bits, "fp8", 80, lambda s, n: list(range(0, n, 16)))
    args = (dev(q), dev(kp), dev(vp, torch.uint8), dev(lay.block_tables), dev(lay.seq_lens))
    say("sparse-V decode, threshold 1e-30 against the exact call")
    for split in (0, 64):
        a = host(pkv.paged_decode_attn(*args, scale=D ** -0.5, k_scale=0.5, v_tq_bits=bits,
                                       split_tokens=split))
        b = host(pkv.paged_decode_attn(*args, scale=D ** -0.5, k_scale=0.5, v_tq_bits=bits,
                                       split_tokens=split, sparse_v_threshold=1e-30))
        err = attn_err(b, a)
        say(f"  split {split}: {err:.3e} from the exact call")
        assert np.isfinite(b).all() and err <= 1e-5


def test_noalloc_call_matches():
    lay = W.layout_for(2, [17, 300, 999])
    Hkv, G, bits = 2, 4, 2
    q, kp, vp = _peaked(lay, Hkv, G, bits, "bf16", 81, lambda s, n: list(range(0, n, 16)))
    args = (dev(q), dev(kp), dev(vp, torch.uint8), dev(lay.block_tables), dev(lay.seq_lens))
    say("sparse-V decode: no-allocation call against the workspace call")
    a = pkv.paged_decode_attn(*args, scale=D ** -0.5, v_tq_bits=bits, sparse_v_threshold=TAU)
    b = torch.full_like(a, float("nan"))
    pkv.paged_decode_attn_noalloc(*args, out=b, scale=D ** -0.5, v_tq_bits=bits,
                                  sparse_v_threshold=TAU)
    assert torch.equal(a, b)
