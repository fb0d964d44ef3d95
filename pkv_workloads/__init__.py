"""Seeded synthetic inputs for the paged KV-cache path.

This module only draws random numbers and lays them out (sequence lengths,
shuffled block tables, K/V/q values, weights, positions).  It holds none of
the method's arithmetic: no normalisation, rotation, quantisation, slot
computation or attention.  Both the CPU oracle's tests and the HIP path's
tests and benchmark draw their inputs from here.

Workloads (one seed per workload, ``seed = 1000 + index``):

0. tiny: 1 sequence of 64 tokens, Hq 4 / Hkv 2, D = R = 64, block 16, pool of
   16 blocks of which 4 (seeded choice) form the block table; K, V, q BF16
   N(0,1); norm weight U(0.5, 1.5); eps 1e-6; theta 1e4; scale 1/8.
1. prefill write: 16 sequences, lengths U{256..1024}, Hkv 8, D = R = 128,
   block 16, pool 1024 blocks in a seeded shuffle; K = BF16(N(0,1) * m_h) with
   m_h = linspace(1, 18, 8) per kv head; V BF16 N(0,1).
2. BF16 decode: 256 sequences, lengths U{512..8192}, Hq 32 / Hkv 8, D 128,
   block 16, pool = sum of ceil(n/16) blocks plus one padding block, shuffled.
3. FP8-K decode: 64 sequences, lengths U{16384..32768}, Hq 64 / Hkv 8, D 128,
   block 16, q and K N(0,1) with 1% of elements times 10, V BF16 N(0,1).
4. gated MLA-style decode: 1 sequence of 4096, 64 heads (MHA), Dqk 192
   (128 NoPE + 64 RoPE), Dv 128, theta 5e4, FP32 q/K/V N(0,1), gate U(0,1).

BF16 values are FP32 draws rounded to nearest even (torch's cast).  Arrays
on the host are numpy (BF16 as uint16 bit patterns); ``device=`` variants
return torch tensors drawn on the device with torch's seeded generator.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

WORKLOADS = {
    0: dict(name="tiny_e2e", num_seqs=1, len_lo=64, len_hi=64, num_q_heads=4, num_kv_heads=2,
            head_dim=64, head_dim_v=64, rotary_dim=64, rope_offset=0, block_size=16,
            theta=10000.0, eps=1e-6, kv_dtype="bf16", k_cache_dtype="bf16"),
    1: dict(name="prefill_write_bf16", num_seqs=16, len_lo=256, len_hi=1024, num_q_heads=8,
            num_kv_heads=8, head_dim=128, head_dim_v=128, rotary_dim=128, rope_offset=0,
            block_size=16, theta=10000.0, eps=1e-6, kv_dtype="bf16", k_cache_dtype="bf16",
            pool_blocks=1024),
    2: dict(name="decode_bf16_256seq", num_seqs=256, len_lo=512, len_hi=8192, num_q_heads=32,
            num_kv_heads=8, head_dim=128, head_dim_v=128, rotary_dim=128, rope_offset=0,
            block_size=16, theta=10000.0, eps=1e-6, kv_dtype="bf16", k_cache_dtype="bf16"),
    3: dict(name="decode_fp8k_64seq_long", num_seqs=64, len_lo=16384, len_hi=32768,
            num_q_heads=64, num_kv_heads=8, head_dim=128, head_dim_v=128, rotary_dim=128,
            rope_offset=0, block_size=16, theta=10000.0, eps=1e-6, kv_dtype="bf16",
            k_cache_dtype="fp8"),
    4: dict(name="gated_mla_f32_4096", num_seqs=1, len_lo=4096, len_hi=4096, num_q_heads=64,
            num_kv_heads=64, head_dim=192, head_dim_v=128, rotary_dim=64, rope_offset=128,
            block_size=16, theta=50000.0, eps=1e-6, kv_dtype="f32", k_cache_dtype="f32"),
}


def seed_of(index: int) -> int:
    return 1000 + index


def rng(index: int, stream: int) -> np.random.Generator:
    """Independent PCG64 sub-stream ``stream`` of workload ``index``."""
    return np.random.default_rng([seed_of(index), stream])


# streams (fixed numbers so that each array is independent of draw order)
S_LENS, S_BLOCKS, S_K, S_V, S_Q, S_W, S_GATE, S_KNEW, S_VNEW, S_POOLK, S_POOLV, S_OUTL, S_SINKS = \
    range(13)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """FP32 draws -> BF16 bit patterns (uint16), round to nearest even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclass
class Layout:
    """Sequence lengths, block tables and pool geometry of one workload."""
    index: int
    seq_lens: np.ndarray            # int32 [S]
    block_tables: np.ndarray        # int32 [S, M]; padding entries = pad_block
    num_blocks: int
    pad_block: int                  # block that padding entries point to (never read)
    block_size: int
    cfg: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.size)

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    @property
    def total_tokens(self) -> int:
        return int(self.seq_lens.astype(np.int64).sum())


def layout(index: int, num_seqs: int | None = None, len_hi: int | None = None) -> Layout:
    """Lengths and shuffled block tables.  ``num_seqs``/``len_hi`` shrink a
    workload for fast tests (the first ``num_seqs`` lengths of the same draw,
    each clipped to ``len_hi``)."""
    cfg = dict(WORKLOADS[index])
    B = cfg["block_size"]
    S_full = cfg["num_seqs"]
    lens = rng(index, S_LENS).integers(cfg["len_lo"], cfg["len_hi"] + 1, size=S_full)
    S = S_full if num_seqs is None else int(num_seqs)
    if S > S_full:
        extra = rng(index, S_LENS + 100).integers(cfg["len_lo"], cfg["len_hi"] + 1,
                                                  size=S - S_full)
        lens = np.concatenate([lens, extra])
    lens = lens[:S]
    if len_hi is not None:
        lens = np.minimum(lens, len_hi)
    lens = lens.astype(np.int32)
    nblk = (lens.astype(np.int64) + B - 1) // B
    M = int(math.ceil(cfg["len_hi"] / B)) if len_hi is None else int(math.ceil(len_hi / B))
    r = rng(index, S_BLOCKS)
    if index == 0:
        # a seeded random choice of 4 distinct blocks out of a pool of 16
        pool = 16
        chosen = r.choice(pool, size=int(nblk[0]), replace=False).astype(np.int32)
        bt = chosen.reshape(1, -1)
        return Layout(index, lens, bt, pool, -1, B, cfg)
    if index == 4:
        # contiguous KV: the identity block table
        pool = int(nblk.sum())
        bt = np.arange(pool, dtype=np.int32).reshape(1, -1)
        return Layout(index, lens, bt, pool, -1, B, cfg)
    used = int(nblk.sum())
    pool = max(cfg.get("pool_blocks", 0), used + 1)
    perm = r.permutation(pool).astype(np.int32)
    pad_block = int(perm[-1])                     # one block kept out of every table
    bt = np.full((S, M), pad_block, np.int32)
    off = 0
    for s in range(S):
        bt[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += int(nblk[s])
    return Layout(index, lens, bt, pool, pad_block, B, cfg)


def layout_for(index: int, lens, max_blocks_per_seq: int | None = None) -> Layout:
    """Block tables (seeded shuffle of a pool sized to fit, plus one padding
    block) for explicitly given sequence lengths."""
    cfg = dict(WORKLOADS[index])
    B = cfg["block_size"]
    lens = np.asarray(lens, np.int32)
    nblk = (np.maximum(lens.astype(np.int64), 0) + B - 1) // B
    M = int(max(1, nblk.max())) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    used = int(nblk.sum())
    pool = used + 1
    perm = rng(index, S_BLOCKS + 200).permutation(pool).astype(np.int32)
    pad_block = int(perm[-1])
    bt = np.full((lens.size, M), pad_block, np.int32)
    off = 0
    for s in range(lens.size):
        bt[s, :nblk[s]] = perm[off:off + nblk[s]]
        off += int(nblk[s])
    return Layout(index, lens, bt, pool, pad_block, B, cfg)


def normal(index: int, stream: int, shape, outliers: bool = False) -> np.ndarray:
    x = rng(index, stream).standard_normal(size=shape, dtype=np.float32)
    if outliers:
        hit = rng(index, stream + 1000).random(size=shape) < 0.01
        x = np.where(hit, x * np.float32(10.0), x)
    return x


def uniform(index: int, stream: int, shape, lo: float, hi: float) -> np.ndarray:
    return rng(index, stream).uniform(lo, hi, size=shape).astype(np.float32)


def norm_weight(index: int) -> np.ndarray:
    """k_norm_weight [D], U(0.5, 1.5), in the K dtype of the workload."""
    cfg = WORKLOADS[index]
    w = uniform(index, S_W, (cfg["head_dim"],), 0.5, 1.5)
    return bf16_bits(w) if cfg["kv_dtype"] == "bf16" else w


def kv_tokens(index: int, num_tokens: int, which: str, stream_base: int | None = None):
    """K or V rows [T, Hkv, D] for ``num_tokens`` tokens (host, numpy)."""
    cfg = WORKLOADS[index]
    H = cfg["num_kv_heads"]
    D = cfg["head_dim"] if which == "k" else cfg["head_dim_v"]
    stream = (S_K if which == "k" else S_V) if stream_base is None else stream_base
    x = normal(index, stream, (num_tokens, H, D), outliers=(index == 3 and which == "k"))
    if index == 1 and which == "k":
        x = x * np.linspace(1.0, 18.0, H, dtype=np.float32)[None, :, None]
    return bf16_bits(x) if cfg["kv_dtype"] == "bf16" else x


def queries(index: int, num_seqs: int) -> np.ndarray:
    cfg = WORKLOADS[index]
    x = normal(index, S_Q, (num_seqs, cfg["num_q_heads"], cfg["head_dim"]),
               outliers=(index == 3))
    return bf16_bits(x) if cfg["kv_dtype"] == "bf16" else x


def gate(index: int, num_seqs: int) -> np.ndarray:
    cfg = WORKLOADS[index]
    return uniform(index, S_GATE, (num_seqs, cfg["num_q_heads"], cfg["head_dim_v"]), 0.0, 1.0)


def positions_all(lay: Layout):
    """Every token of every sequence, positions 0..n-1: (start_pos, cu_counts, pos)."""
    lens = lay.seq_lens.astype(np.int64)
    cu = np.zeros(lay.num_seqs + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    start = np.zeros(lay.num_seqs, np.int32)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens]) if lay.num_seqs else \
        np.zeros(0, np.int32)
    return start, cu, pos


def positions_history(lay: Layout):
    """All tokens but the last of each sequence (the decode history)."""
    lens = np.maximum(lay.seq_lens.astype(np.int64) - 1, 0)
    cu = np.zeros(lay.num_seqs + 1, np.int64)
    cu[1:] = np.cumsum(lens)
    start = np.zeros(lay.num_seqs, np.int32)
    pos = np.concatenate([np.arange(n, dtype=np.int32) for n in lens])
    return start, cu, pos


def positions_decode(lay: Layout):
    """The last token of each sequence (position n-1), one per sequence."""
    start = (lay.seq_lens.astype(np.int64) - 1).astype(np.int32)
    cu = np.arange(lay.num_seqs + 1, dtype=np.int64)
    return start, cu, start.copy()


def e4m3_codes(index: int, stream: int, shape) -> np.ndarray:
    """Random finite E4M3 codes with exponent field <= 9 (|value| <= 7.5),
    random sign."""
    r = rng(index, stream)
    mag = r.integers(0, 0x50, size=shape).astype(np.uint8)
    sign = (r.integers(0, 2, size=shape).astype(np.uint8) << 7).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def e4m3_finite_codes(index: int, stream: int, shape) -> np.ndarray:
    """Random finite E4M3 codes over the whole range: magnitude codes
    0x00..0x7E (0 to 448: every exponent field, subnormals included), random
    sign."""
    r = rng(index, stream)
    mag = r.integers(0, 0x7F, size=shape).astype(np.uint8)
    sign = (r.integers(0, 2, size=shape).astype(np.uint8) << 7).astype(np.uint8)
    return (mag | sign).astype(np.uint8)


def random_pools(index: int, lay: Layout, poison_pad: bool = True, v_dtype: str = None):
    """K and V pools [num_blocks, B, Hkv, D] filled directly with random
    values (decode tested on its own).  K is N(0,1) (BF16 or FP32; the FP8
    pool holds random finite E4M3 codes); V likewise, or E4M3 codes with
    ``v_dtype="fp8"``; with ``poison_pad`` the padding block is NaN.
    Returns (k_pool, v_pool) as numpy arrays."""
    cfg = WORKLOADS[index]
    H, D, Dv, B = cfg["num_kv_heads"], cfg["head_dim"], cfg["head_dim_v"], cfg["block_size"]
    kshape = (lay.num_blocks, B, H, D)
    vshape = (lay.num_blocks, B, H, Dv)
    if cfg["k_cache_dtype"] == "fp8":
        kp = e4m3_codes(index, S_POOLK, kshape)
    else:
        kx = normal(index, S_POOLK, kshape, outliers=(index == 3))
        kp = bf16_bits(kx) if cfg["k_cache_dtype"] == "bf16" else kx
    if v_dtype == "fp8":
        vp = e4m3_codes(index, S_POOLV, vshape)
    else:
        vx = normal(index, S_POOLV, vshape)
        vp = bf16_bits(vx) if cfg["kv_dtype"] == "bf16" else vx
    if poison_pad and lay.pad_block >= 0:
        if kp.dtype == np.uint8:
            kp[lay.pad_block] = 0x7F
        elif kp.dtype == np.uint16:
            kp[lay.pad_block] = 0x7FC0
        else:
            kp[lay.pad_block] = np.nan
        if vp.dtype == np.uint8:
            vp[lay.pad_block] = 0x7F
        elif vp.dtype == np.uint16:
            vp[lay.pad_block] = 0x7FC0
        else:
            vp[lay.pad_block] = np.nan
    return kp, vp


# --------------------------------------------------------------------------
# device-side draws for full-size workloads (torch, seeded)
# --------------------------------------------------------------------------

def device_normal(index: int, stream: int, shape, dtype, device, outliers=False,
                  scale_per_head=None, chunk_rows: int = 1 << 16):
    """N(0,1) draws made on the device with torch's seeded generator, cast to
    ``dtype`` (a torch dtype).  Drawn in row chunks to bound temporaries."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(index) * 1000 + stream)
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(shape[0], -1)
    for r0 in range(0, shape[0], chunk_rows):
        r1 = min(shape[0], r0 + chunk_rows)
        x = torch.randn((r1 - r0, flat.shape[1]), generator=g, device=device,
                        dtype=torch.float32)
        if outliers:
            hit = torch.rand(x.shape, generator=g, device=device) < 0.01
            x = torch.where(hit, x * 10.0, x)
        if scale_per_head is not None:
            x = (x.view(r1 - r0, len(scale_per_head), -1) *
                 torch.tensor(scale_per_head, device=device).view(1, -1, 1)).view(x.shape)
        flat[r0:r1] = x.to(dtype)
        del x
    return out
