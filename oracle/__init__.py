"""CPU oracle for the paged KV-cache path -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes wrapper around ``pkv_oracle.c`` (plain C, FP64, scalar).
Only the test suite, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg may import this package.  The product library never
imports it and shares no code with it.

Array conventions (all numpy, C-contiguous):
  * BF16 data is carried as ``np.uint16`` bit patterns,
  * E4M3 (OCP FP8 E4M3FN) data as ``np.uint8`` codes,
  * FP32 data as ``np.float32``.
Dtype names: ``"bf16"``, ``"fp8"``, ``"f32"``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkv_oracle.so")
SRC_PATH = os.path.join(_HERE, "pkv_oracle.c")

DTYPES = {"bf16": 0, "fp8": 1, "f32": 2, "tq2": 3, "tq3": 4, "tq4": 5}
NP_TYPES = {"bf16": np.uint16, "fp8": np.uint8, "f32": np.float32, "tq2": np.uint8,
            "tq3": np.uint8, "tq4": np.uint8}


def build() -> str:
    """Compile the oracle with gcc (plain C11, no fast-math, no contraction)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-std=c11", "-Wall", "-fPIC", "-shared",
           SRC_PATH, "-o", LIB_PATH, "-lm", "-pthread"]
    subprocess.run(cmd, check=True)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, U32, U64, I32, F32 = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                                 ctypes.c_int, ctypes.c_float)
        L.pkvo_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.pkvo_f32_from_bf16.restype = ctypes.c_float
        L.pkvo_bf16_from_f32.argtypes = [F32]
        L.pkvo_bf16_from_f32.restype = ctypes.c_uint16
        L.pkvo_f64_from_e4m3.argtypes = [ctypes.c_uint8]
        L.pkvo_f64_from_e4m3.restype = ctypes.c_double
        L.pkvo_e4m3_from_f64.argtypes = [ctypes.c_double]
        L.pkvo_e4m3_from_f64.restype = ctypes.c_uint8
        L.pkvo_rope_inv_freq.argtypes = [F32, U32, U32]
        L.pkvo_rope_inv_freq.restype = F32
        L.pkvo_rope_angle.argtypes = [ctypes.c_int32, F32]
        L.pkvo_rope_angle.restype = F32
        for name in ("pkvo_bf16_from_f32_array", "pkvo_e4m3_from_f32_array",
                     "pkvo_f64_from_e4m3_array"):
            getattr(L, name).argtypes = [P, P, U64]
            getattr(L, name).restype = None
        L.pkvo_fill_slots.argtypes = [P, P, U32, P, P, U32, U32, U32]
        L.pkvo_fill_slots.restype = None
        L.pkvo_cache_write_k.argtypes = [P, I32, U64, P, F32, P, P, P, F32, U32, U32, I32,
                                         P, U32, U32, U32, U32, U32, P, I32, F32, I32]
        L.pkvo_cache_write_k.restype = None
        L.pkvo_cache_write_v.argtypes = [P, I32, U64, P, U32, U32, U32, U32, U32, P, I32, F32]
        L.pkvo_cache_write_v.restype = None
        L.pkvo_paged_decode.argtypes = [P, I32, U64, P, I32, F32, P, I32, F32, P, U32, P, U32,
                                        U32, U32, U32, U32, U32, U32, F32, U32, P, I32, F32,
                                        U32, U32, P, P, I32]
        L.pkvo_paged_decode.restype = None
        L.pkvo_paged_decode_sparse_v.argtypes = [P, I32, U64, P, I32, F32, P, I32, F32, P, U32,
                                                 P, U32, U32, U32, U32, U32, U32, U32, F32, U32,
                                                 P, P, ctypes.c_double, P, P, I32]
        L.pkvo_paged_decode_sparse_v.restype = None
        L.pkvo_paged_prefill.argtypes = [P, I32, U64, P, P, I32, F32, P, I32, F32, P, U32, P, U32,
                                         U32, U32, U32, U32, U32, U32, F32, U32, P, P, I32]
        L.pkvo_paged_prefill.restype = None
        L.pkvo_tq_lloyd_max.argtypes = [I32, P]
        L.pkvo_tq_lloyd_max.restype = None
        L.pkvo_tq_codebook.argtypes = [I32, P]
        L.pkvo_tq_codebook.restype = None
        L.pkvo_tq_block_bytes.argtypes = [I32, U32, U32, U32]
        L.pkvo_tq_block_bytes.restype = U64
        L.pkvo_tq_encode_diag.argtypes = [P, I32, U64, U32, U32, U32, I32, P, P, P, P, P]
        L.pkvo_tq_encode_diag.restype = None
        L.pkvo_mla_cache_assemble.argtypes = [P, P, I32, U64, U64, P, U32, U32, U32, U32, U32,
                                              U32, P, P]
        L.pkvo_mla_cache_assemble.restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """C-contiguous array of the given numpy dtype (no copy when already so)."""
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def bf16_from_f32(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, np.uint16)
    lib().pkvo_bf16_from_f32_array(_ptr(x), _ptr(out), x.size)
    return out


def f32_from_bf16(h) -> np.ndarray:
    h = np.asarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


def e4m3_from_f32(x) -> np.ndarray:
    x = _c(np.asarray(x, dtype=np.float32), np.float32)
    out = np.empty(x.shape, np.uint8)
    lib().pkvo_e4m3_from_f32_array(_ptr(x), _ptr(out), x.size)
    return out


def f64_from_e4m3(c) -> np.ndarray:
    c = _c(np.asarray(c, dtype=np.uint8), np.uint8)
    out = np.empty(c.shape, np.float64)
    lib().pkvo_f64_from_e4m3_array(_ptr(c), _ptr(out), c.size)
    return out


def rope_inv_freq(theta: float, i: int, rotary_dim: int) -> float:
    return float(lib().pkvo_rope_inv_freq(theta, i, rotary_dim))


def rope_angle(pos: int, inv_freq: float) -> float:
    return float(lib().pkvo_rope_angle(pos, inv_freq))


def to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact FP64 value of stored data (FP8 without scale)."""
    if dtype == "bf16":
        return f32_from_bf16(a).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, np.float32).astype(np.float64)
    return f64_from_e4m3(a)


# --------------------------------------------------------------------------
# the four operations
# --------------------------------------------------------------------------

def fill_slots(block_tables, start_pos, cu_counts, total_tokens: int, block_size: int):
    """Slots (int64 [total_tokens]) of the batched token ranges."""
    bt = _c(block_tables, np.int32)
    if bt.ndim == 1:
        bt = bt.reshape(1, -1)
    sp = _c(start_pos, np.int32)
    cu = _c(cu_counts, np.int64).astype(np.int32)
    out = np.empty(total_tokens, np.int64)
    lib().pkvo_fill_slots(_ptr(out), _ptr(bt), bt.shape[1], _ptr(sp), _ptr(cu), sp.size,
                          total_tokens, block_size)
    return out


def cache_write_k(k_in, in_dtype, slots, k_cache, cache_dtype, *, num_kv_heads, head_dim,
                  block_size, norm_weight=None, eps=1e-6, pos_t=None, pos_h=None, pos_w=None,
                  theta=10000.0, rope_offset=0, rotary_dim=None, nope=False, k_scale=1.0,
                  in_token_stride=None, nthreads=1):
    """Fused K write into ``k_cache`` (modified in place).

    ``k_in``: [T, Hkv, D] (or a 2-D [T, stride] view) of ``in_dtype``;
    ``k_cache``: [num_blocks, block_size, Hkv, D] of ``cache_dtype``.
    """
    k_in = _c(k_in, NP_TYPES[in_dtype])
    T = int(slots.size)
    stride = in_token_stride if in_token_stride is not None else num_kv_heads * head_dim
    assert k_cache.flags.c_contiguous and k_cache.dtype == NP_TYPES[cache_dtype]
    num_blocks = k_cache.size // (block_size * num_kv_heads * head_dim)
    if rotary_dim is None:
        rotary_dim = head_dim
    w = _c(norm_weight, NP_TYPES[in_dtype])
    pt = _c(pos_t, np.int32) if pos_t is not None else np.zeros(T, np.int32)
    ph = _c(pos_h, np.int32)
    pw = _c(pos_w, np.int32)
    sl = _c(slots, np.int64)
    lib().pkvo_cache_write_k(_ptr(k_in), DTYPES[in_dtype], stride, _ptr(w), eps, _ptr(pt),
                             _ptr(ph), _ptr(pw), theta, rope_offset, rotary_dim, int(nope),
                             _ptr(sl), T, num_kv_heads, head_dim, block_size, num_blocks,
                             _ptr(k_cache), DTYPES[cache_dtype], k_scale, nthreads)
    return k_cache


def cache_write_v(v, dtype, slots, v_cache, *, num_kv_heads, head_dim_v, block_size,
                  in_token_stride=None, cache_dtype=None, v_scale=1.0):
    """V rows into ``v_cache`` (modified in place): a byte copy when the cache
    has the input's dtype, else (``cache_dtype="fp8"``) E4M3 of v / v_scale."""
    cache_dtype = cache_dtype or dtype
    v = _c(v, NP_TYPES[dtype])
    T = int(slots.size)
    stride = in_token_stride if in_token_stride is not None else num_kv_heads * head_dim_v
    assert v_cache.flags.c_contiguous and v_cache.dtype == NP_TYPES[cache_dtype]
    if cache_dtype.startswith("tq"):
        num_blocks = v_cache.size // tq_block_bytes(int(cache_dtype[2]), block_size, num_kv_heads,
                                                    head_dim_v)
    else:
        num_blocks = v_cache.size // (block_size * num_kv_heads * head_dim_v)
    sl = _c(slots, np.int64)
    lib().pkvo_cache_write_v(_ptr(v), DTYPES[dtype], stride, _ptr(sl), T, num_kv_heads,
                             head_dim_v, block_size, num_blocks, _ptr(v_cache),
                             DTYPES[cache_dtype], v_scale)
    return v_cache


def paged_decode(q, q_dtype, k_cache, k_dtype, v_cache, v_dtype, block_tables, seq_lens, *,
                 num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, block_size, scale,
                 k_scale=1.0, v_scale=1.0, sliding_window=0, sinks=None, q_rope=False,
                 q_rope_theta=10000.0, q_rope_offset=0, q_rope_dim=0, gate=None,
                 q_seq_stride=None, nthreads=1):
    """Decode attention, one query token per sequence.  Returns FP32
    [num_seqs, num_q_heads, head_dim_v]."""
    q = _c(q, NP_TYPES[q_dtype])
    bt = _c(block_tables, np.int32)
    if bt.ndim == 1:
        bt = bt.reshape(1, -1)
    sl = _c(seq_lens, np.int32)
    S = sl.size
    kc = _c(k_cache, NP_TYPES[k_dtype])
    vc = _c(v_cache, NP_TYPES[v_dtype])
    num_blocks = kc.size // (block_size * num_kv_heads * head_dim_qk)
    qs = q_seq_stride if q_seq_stride is not None else num_q_heads * head_dim_qk
    g = _c(gate, np.float32)
    sk = _c(sinks, np.float32)
    out = np.empty((S, num_q_heads, head_dim_v), np.float32)
    lib().pkvo_paged_decode(_ptr(q), DTYPES[q_dtype], qs, _ptr(kc), DTYPES[k_dtype], k_scale,
                            _ptr(vc), DTYPES[v_dtype], v_scale, _ptr(bt), bt.shape[1], _ptr(sl),
                            S, num_blocks, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v,
                            block_size, scale, sliding_window, _ptr(sk), int(q_rope),
                            q_rope_theta, q_rope_offset,
                            q_rope_dim, _ptr(g), _ptr(out), nthreads)
    return out


def paged_decode_sparse_v(q, q_dtype, k_cache, k_dtype, v_cache, v_dtype, block_tables,
                          seq_lens, *, num_q_heads, num_kv_heads, head_dim_qk, head_dim_v,
                          block_size, scale, tau, k_scale=1.0, v_scale=1.0, sliding_window=0,
                          sinks=None, gate=None, nthreads=1):
    """Decode attention with the sparse-V skip at threshold ``tau``: returns
    (out, bound), FP32 [num_seqs, num_q_heads, head_dim_v] each.  ``out`` sums
    w_t v_t over the positions whose softmax weight w_t exceeds tau, ``bound``
    sums w_t |v_t| over the others (times the gate, |gate|), so that any
    decode skipping a subset of the latter lies within ``bound`` of ``out``."""
    q = _c(q, NP_TYPES[q_dtype])
    bt = _c(block_tables, np.int32)
    if bt.ndim == 1:
        bt = bt.reshape(1, -1)
    sl = _c(seq_lens, np.int32)
    S = sl.size
    kc = _c(k_cache, NP_TYPES[k_dtype])
    vc = _c(v_cache, NP_TYPES[v_dtype])
    num_blocks = kc.size // (block_size * num_kv_heads * head_dim_qk)
    g = _c(gate, np.float32)
    sk = _c(sinks, np.float32)
    out = np.empty((S, num_q_heads, head_dim_v), np.float32)
    bound = np.empty_like(out)
    lib().pkvo_paged_decode_sparse_v(_ptr(q), DTYPES[q_dtype], num_q_heads * head_dim_qk,
                                     _ptr(kc), DTYPES[k_dtype], k_scale, _ptr(vc),
                                     DTYPES[v_dtype], v_scale, _ptr(bt), bt.shape[1], _ptr(sl),
                                     S, num_blocks, num_q_heads, num_kv_heads, head_dim_qk,
                                     head_dim_v, block_size, scale, sliding_window, _ptr(sk),
                                     _ptr(g), float(tau), _ptr(out), _ptr(bound), nthreads)
    return out, bound


def paged_prefill(q, q_dtype, cu_q, k_cache, k_dtype, v_cache, v_dtype, block_tables, seq_lens, *,
                  num_q_heads, num_kv_heads, head_dim_qk, head_dim_v, block_size, scale,
                  k_scale=1.0, v_scale=1.0, sliding_window=0, sinks=None, q_token_stride=None,
                  nthreads=1):
    """Causal attention of the last q_len tokens of every sequence over the
    paged cache.  q [total_q, Hq, Dqk]; cu_q int32 [S+1].  Returns FP32
    [total_q, num_q_heads, head_dim_v]."""
    q = _c(q, NP_TYPES[q_dtype])
    cq = _c(cu_q, np.int32)
    bt = _c(block_tables, np.int32)
    if bt.ndim == 1:
        bt = bt.reshape(1, -1)
    sl = _c(seq_lens, np.int32)
    S = sl.size
    kc = _c(k_cache, NP_TYPES[k_dtype])
    vc = _c(v_cache, NP_TYPES[v_dtype])
    num_blocks = kc.size // (block_size * num_kv_heads * head_dim_qk)
    qs = q_token_stride if q_token_stride is not None else num_q_heads * head_dim_qk
    total = int(cq[S]) if S else 0
    sk = _c(sinks, np.float32)
    out = np.empty((total, num_q_heads, head_dim_v), np.float32)
    lib().pkvo_paged_prefill(_ptr(q), DTYPES[q_dtype], qs, _ptr(cq), _ptr(kc), DTYPES[k_dtype],
                             k_scale, _ptr(vc), DTYPES[v_dtype], v_scale, _ptr(bt), bt.shape[1],
                             _ptr(sl), S, num_blocks, num_q_heads, num_kv_heads, head_dim_qk,
                             head_dim_v, block_size, scale, sliding_window, _ptr(sk), _ptr(out),
                             nthreads)
    return out


def mla_cache_assemble(kv_latent, k_rope, dtype, slots, k_cache, v_cache, *, kv_lora, rope,
                            block_size, latent_stride=None, rope_stride=None):
    """K row [latent | k_rope | 0], V row [latent | 0] at every slot (caches
    [num_blocks, block_size, 1, cache_dim], modified in place).  kv_latent
    [T, >= kv_lora] and k_rope [T, >= rope] with token strides."""
    lat = _c(kv_latent, NP_TYPES[dtype])
    rp = _c(k_rope, NP_TYPES[dtype])
    T = int(slots.size)
    ls = latent_stride if latent_stride is not None else lat.shape[-1]
    rs = rope_stride if rope_stride is not None else rp.shape[-1]
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    assert k_cache.dtype == NP_TYPES[dtype] and v_cache.dtype == NP_TYPES[dtype]
    cache_dim = k_cache.shape[-1]
    num_blocks = k_cache.size // (block_size * cache_dim)
    sl = _c(slots, np.int64)
    lib().pkvo_mla_cache_assemble(_ptr(lat), _ptr(rp), DTYPES[dtype], ls, rs, _ptr(sl), T,
                                  kv_lora, rope, cache_dim, block_size, num_blocks,
                                  _ptr(k_cache), _ptr(v_cache))
    return k_cache, v_cache


def tq_lloyd_max(bits: int) -> np.ndarray:
    """The 2^bits Lloyd-Max levels of N(0,1), ascending (FP64)."""
    out = np.empty(1 << bits, np.float64)
    lib().pkvo_tq_lloyd_max(bits, _ptr(out))
    return out


def tq_codebook(bits: int) -> np.ndarray:
    """E4M3 codes of the positive codebook magnitudes, ascending."""
    out = np.empty(1 << (bits - 1), np.uint8)
    lib().pkvo_tq_codebook(bits, _ptr(out))
    return out


def tq_block_bytes(bits: int, block_size: int, num_kv_heads: int, head_dim_v: int) -> int:
    return int(lib().pkvo_tq_block_bytes(bits, block_size, num_kv_heads, head_dim_v))


def tq_encode_diag(v, dtype, bits: int, *, num_kv_heads, head_dim_v, in_token_stride=None):
    """What the TQ encoder decides each group from, for rows v [T, H, D]:
    returns (u [T, H, D] = x / rms, ss [T, H, D/16] = sum of squares, ratio
    [T, H, D/16] = |x| / |chosen levels|, codes [T, H, D] = sign << (b-1) |
    magnitude index, scales [T, H, D/16] E4M3 bytes), FP64 / uint8."""
    v = _c(v, NP_TYPES[dtype])
    T = v.shape[0]
    H, D = num_kv_heads, head_dim_v
    stride = in_token_stride if in_token_stride is not None else H * D
    u = np.empty((T, H, D), np.float64)
    ss = np.empty((T, H, D // 16), np.float64)
    ratio = np.empty((T, H, D // 16), np.float64)
    codes = np.empty((T, H, D), np.uint8)
    scales = np.empty((T, H, D // 16), np.uint8)
    lib().pkvo_tq_encode_diag(_ptr(v), DTYPES[dtype], stride, T, H, D, bits, _ptr(u), _ptr(ss),
                              _ptr(ratio), _ptr(codes), _ptr(scales))
    return u, ss, ratio, codes, scales
