"""paged_kv_cache_fill_amd -- Python binding of libpkv (MI355X / gfx950).

Thin ctypes marshalling over the C ABI declared in ``include/pkv.h``: every
function takes torch tensors that already live on the GPU, checks dtypes,
shapes and contiguity, and passes raw pointers, sizes and the current HIP
stream to the library.  All computation happens in the library's HIP kernels;
there is no fallback path.  If the library is not built, importing works but
every call raises ``RuntimeError``.

Functions (same names as the C calls without the ``pkv_`` prefix):
  fill_slots, cache_write_k_fused, cache_write_v, decode_workspace_bytes,
  paged_decode_attn, paged_decode_attn_noalloc, paged_prefill_attn, mla_cache_assemble
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["fill_slots", "cache_write_k_fused", "cache_write_v", "decode_workspace_bytes",
           "paged_decode_attn", "paged_decode_attn_noalloc", "paged_prefill_attn", "mla_cache_assemble", "v_block_bytes",
           "tq_codebook", "library_path", "load", "PkvError"]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpkv.so")

BF16, FP8_E4M3, FP32 = 0, 1, 2
DECODE_SCRATCH_BYTES = 32 << 20          # PKV_DECODE_SCRATCH_BYTES
TQ2, TQ3, TQ4 = 3, 4, 5                  # TurboQuant-style V cache formats (see pkv.h)
_DT = {torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3, torch.uint8: FP8_E4M3,
       torch.float32: FP32}

_P, _U32, _U64, _I32, _F32, _SZ = (ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64,
                                   ctypes.c_int, ctypes.c_float, ctypes.c_size_t)
_SIGNATURES = {
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_version": ([], ctypes.c_char_p),
    "pkv_fill_slots": ([_P, _P, _U32, _P, _P, _U32, _U32, _U32, _P], _I32),
    "pkv_cache_write_k_fused": ([_P, _I32, _U64, _P, _F32, _P, _P, _P, _F32, _U32, _U32, _I32,
                                 _P, _U32, _U32, _U32, _U32, _U32, _P, _I32, _F32, _P], _I32),
    "pkv_cache_write_v": ([_P, _I32, _U64, _P, _U32, _U32, _U32, _U32, _U32, _P, _I32, _F32,
                           _P], _I32),
    "pkv_decode_workspace_bytes": ([_U32, _U32, _U32, _U32, _U32, _U32, _U32, _U32], _SZ),
    "pkv_paged_decode_attn": ([_P, _I32, _U64, _P, _I32, _F32, _P, _I32, _F32, _F32, _P, _U32,
                               _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _F32, _U32, _P,
                               _I32, _F32, _U32, _U32, _P, _P, _U32, _P, _SZ, _P], _I32),
    "pkv_paged_decode_attn_noalloc": ([_P, _I32, _U64, _P, _I32, _F32, _P, _I32, _F32, _F32, _P,
                                       _U32, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _F32,
                                       _U32, _P, _I32, _F32, _U32, _U32, _P, _P, _U32, _P], _I32),
    "pkv_paged_prefill_attn": ([_P, _I32, _U64, _P, _U32, _U32, _P, _I32, _F32, _P, _I32, _F32,
                                _P, _U32, _P, _U32, _U32, _U32, _U32, _U32, _U32, _U32, _F32,
                                _U32, _P, _P, _P], _I32),
    "pkv_mla_cache_assemble": ([_P, _P, _I32, _U64, _U64, _P, _U32, _U32, _U32, _U32, _U32, _U32,
                                _P, _P, _P], _I32),
    "pkv_v_block_bytes": ([_I32, _U32, _U32, _U32], _SZ),
    "pkv_tq_codebook": ([_I32, _P], _I32),
}


class PkvError(RuntimeError):
    """A non-zero status from libpkv (message from pkv_last_error)."""

    def __init__(self, status: int, message: str):
        super().__init__(f"libpkv status {status}: {message}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load():
    """Loads libpkv.so (raises RuntimeError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"libpkv.so is not built ({_LIB_PATH}); run "
                               "__graft_entry__.build() or python paged_kv_cache_fill_amd/_build.py")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise PkvError(status, load().pkv_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(*tensors):
    for t in tensors:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _dtype(t):
    try:
        return _DT[t.dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {t.dtype}") from None


def _token_stride(x, name):
    """Token stride (elements) of a [T, H, D] tensor whose heads are packed."""
    if x.dim() != 3:
        raise ValueError(f"{name} must be [tokens, heads, head_dim]")
    if x.stride(2) != 1 or x.stride(1) != x.shape[2]:
        raise ValueError(f"{name}: heads and head_dim must be packed (stride 1, head_dim)")
    return x.stride(0) if x.shape[0] > 1 else x.shape[1] * x.shape[2]


def _pool(cache, name):
    if cache.dim() != 4 or not cache.is_contiguous():
        raise ValueError(f"{name} must be a contiguous [num_blocks, block_size, heads, head_dim] pool")
    return cache.shape


# ---------------------------------------------------------------------------


def fill_slots(slots, block_tables, start_pos, cu_counts, block_size: int):
    """slots[i] for the batched token ranges (see pkv_fill_slots).

    slots int64 [T]; block_tables int32 [S, M]; start_pos int32 [S];
    cu_counts int32 [S+1].
    """
    _dev(slots, block_tables, start_pos, cu_counts)
    if slots.dtype != torch.int64 or block_tables.dtype != torch.int32 or \
            start_pos.dtype != torch.int32 or cu_counts.dtype != torch.int32:
        raise ValueError("slots int64, block_tables/start_pos/cu_counts int32")
    if not (slots.is_contiguous() and block_tables.is_contiguous() and start_pos.is_contiguous()
            and cu_counts.is_contiguous()):
        raise ValueError("fill_slots: tensors must be contiguous")
    S = start_pos.numel()
    if cu_counts.numel() != S + 1 or (S and block_tables.dim() != 2) or \
            (S and block_tables.shape[0] != S):
        raise ValueError("fill_slots: block_tables [S, M], start_pos [S], cu_counts [S+1]")
    M = block_tables.shape[1] if S else 1
    _check(load().pkv_fill_slots(_ptr(slots), _ptr(block_tables), M, _ptr(start_pos),
                                 _ptr(cu_counts), S, slots.numel(), block_size, _stream()))
    return slots


def cache_write_k_fused(k_in, slot_mapping, k_cache, *, norm_weight=None, eps: float = 1e-6,
                        pos_t=None, pos_h=None, pos_w=None, theta: float = 10000.0,
                        rope_offset: int = 0, rotary_dim: int | None = None, nope: bool = False,
                        k_scale: float = 1.0):
    """Fused RMSNorm -> RoPE -> one rounding into the K pool (pkv_cache_write_k_fused).

    k_in [T, Hkv, D] (BF16/FP32, token stride free); slot_mapping int64 [T];
    k_cache [num_blocks, block_size, Hkv, D] (BF16, FP8 E4M3 as float8_e4m3fn or
    uint8, or FP32).
    """
    _dev(k_in, slot_mapping, k_cache, norm_weight, pos_t, pos_h, pos_w)
    nb, B, H, D = _pool(k_cache, "k_cache")
    T = k_in.shape[0]
    if k_in.shape[1:] != (H, D) or slot_mapping.numel() != T or slot_mapping.dtype != torch.int64:
        raise ValueError("k_in [T, Hkv, D] must match the pool; slot_mapping int64 [T]")
    if norm_weight is not None and (norm_weight.numel() != D or norm_weight.dtype != k_in.dtype
                                    or not norm_weight.is_contiguous()):
        raise ValueError("norm_weight must be [D] contiguous of k_in's dtype")
    for p in (pos_t, pos_h, pos_w):
        if p is not None and (p.dtype != torch.int32 or p.numel() != T or not p.is_contiguous()):
            raise ValueError("positions must be int32 [T] contiguous")
    stride = _token_stride(k_in, "k_in")
    R = D if rotary_dim is None else rotary_dim
    _check(load().pkv_cache_write_k_fused(
        _ptr(k_in), _dtype(k_in), stride, _ptr(norm_weight), eps, _ptr(pos_t), _ptr(pos_h),
        _ptr(pos_w), theta, rope_offset, R, int(bool(nope)), _ptr(slot_mapping), T, H, D, B, nb,
        _ptr(k_cache), _dtype(k_cache), k_scale, _stream()))
    return k_cache


def v_block_bytes(v_dtype: int, block_size: int, num_kv_heads: int, head_dim_v: int) -> int:
    """Bytes of one V cache block in the given format (pkv_v_block_bytes)."""
    return int(load().pkv_v_block_bytes(v_dtype, block_size, num_kv_heads, head_dim_v))


def tq_codebook(tq_bits: int):
    """E4M3 codes of a TQ format's positive codebook magnitudes (pkv_tq_codebook)."""
    out = (ctypes.c_uint8 * 8)()
    _check(load().pkv_tq_codebook(tq_bits + 1, out))
    return bytes(out[:1 << (tq_bits - 1)])


def _tq_pool(v_cache, tq_bits, block_size, H, D):
    if v_cache.dtype != torch.uint8 or v_cache.dim() != 2 or not v_cache.is_contiguous():
        raise ValueError("a TQ V pool is a contiguous uint8 [num_blocks, block_bytes] tensor")
    if v_cache.shape[1] != v_block_bytes(tq_bits + 1, block_size, H, D):
        raise ValueError("TQ V pool rows must be v_block_bytes(...) long")
    return v_cache.shape[0]


def cache_write_v(v, slot_mapping, v_cache, v_scale: float = 1.0, tq_bits: int = 0,
                  block_size: int = 16):
    """V rows into the V pool at their slots (pkv_cache_write_v): a byte copy
    when the pool has v's dtype, E4M3 of v / v_scale for an FP8 pool, or the
    TurboQuant-style b-bit format when ``tq_bits`` is 2, 3 or 4 (v_cache a
    uint8 [num_blocks, block_bytes] tensor)."""
    _dev(v, slot_mapping, v_cache)
    T = v.shape[0]
    if tq_bits:
        if v.dim() != 3:
            raise ValueError("v must be [T, Hkv, Dv]")
        H, D = v.shape[1], v.shape[2]
        nb, B = _tq_pool(v_cache, tq_bits, block_size, H, D), block_size
        if slot_mapping.numel() != T or slot_mapping.dtype != torch.int64:
            raise ValueError("slot_mapping must be int64 [T]")
        stride = _token_stride(v, "v")
        _check(load().pkv_cache_write_v(_ptr(v), _dtype(v), stride, _ptr(slot_mapping), T, H, D,
                                        B, nb, _ptr(v_cache), tq_bits + 1, v_scale, _stream()))
        return v_cache
    nb, B, H, D = _pool(v_cache, "v_cache")
    if v.shape[1:] != (H, D):
        raise ValueError("v [T, Hkv, Dv] must match the pool's shape")
    if slot_mapping.numel() != T or slot_mapping.dtype != torch.int64:
        raise ValueError("slot_mapping must be int64 [T]")
    stride = _token_stride(v, "v")
    _check(load().pkv_cache_write_v(_ptr(v), _dtype(v), stride, _ptr(slot_mapping), T, H, D, B,
                                    nb, _ptr(v_cache), _dtype(v_cache), v_scale, _stream()))
    return v_cache


def decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim_v, max_blocks_per_seq,
                           block_size=16, split_tokens=0, sliding_window=0) -> int:
    return int(load().pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads,
                                                 head_dim_v, max_blocks_per_seq, block_size,
                                                 sliding_window, split_tokens))


def _decode_args(q, k_cache, v_cache, block_tables, seq_lens, *, scale, k_scale, v_scale,
                 sparse_v_threshold, sliding_window, sinks, gate, out, q_rope, q_rope_theta,
                 q_rope_offset, q_rope_dim, split_tokens, v_tq_bits, alloc_out):
    """Checks the decode arguments; returns (leading C arguments up to and
    including split_tokens, out, (S, Hq, Hkv, Dv, M, B))."""
    _dev(q, k_cache, v_cache, block_tables, seq_lens, sinks, gate, out)
    nb, B, Hkv, Dqk = _pool(k_cache, "k_cache")
    if v_tq_bits:
        Dv = Dqk
        if _tq_pool(v_cache, v_tq_bits, B, Hkv, Dv) != nb:
            raise ValueError("K and V pools must have the same blocks")
        v_dt = v_tq_bits + 1
    else:
        nb2, B2, Hkv2, Dv = _pool(v_cache, "v_cache")
        if (nb2, B2, Hkv2) != (nb, B, Hkv):
            raise ValueError("K and V pools must have the same blocks and heads")
        v_dt = _dtype(v_cache)
    if q.dim() != 3 or q.shape[2] != Dqk or q.stride(2) != 1 or q.stride(1) != Dqk:
        raise ValueError("q must be [S, Hq, Dqk] with packed heads")
    S, Hq = q.shape[0], q.shape[1]
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != S or not block_tables.is_contiguous():
        raise ValueError("block_tables must be int32 [S, M] contiguous")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != S or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be int32 [S] contiguous")
    if gate is not None and (gate.dtype != torch.float32 or gate.shape != (S, Hq, Dv) or
                             not gate.is_contiguous()):
        raise ValueError("gate must be FP32 [S, Hq, Dv] contiguous")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != Hq or
                              not sinks.is_contiguous()):
        raise ValueError("sinks must be FP32 [Hq] contiguous")
    if out is None:
        if not alloc_out:
            raise ValueError("out must be given (FP32 [S, Hq, Dv])")
        out = torch.empty((S, Hq, Dv), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != (S, Hq, Dv) or not out.is_contiguous():
        raise ValueError("out must be FP32 [S, Hq, Dv] contiguous")
    M = block_tables.shape[1]
    q_stride = q.stride(0) if S > 1 else Hq * Dqk
    args = (_ptr(q), _dtype(q), q_stride, _ptr(k_cache), _dtype(k_cache), k_scale,
            _ptr(v_cache), v_dt, v_scale, sparse_v_threshold, _ptr(block_tables), M,
            _ptr(seq_lens), S, nb, Hq, Hkv,
            Dqk, Dv, B, scale, sliding_window, _ptr(sinks), int(bool(q_rope)), q_rope_theta,
            q_rope_offset, q_rope_dim, _ptr(gate), _ptr(out), split_tokens)
    return args, out, (S, Hq, Hkv, Dv, M, B)


def paged_decode_attn(q, k_cache, v_cache, block_tables, seq_lens, *, scale: float,
                      k_scale: float = 1.0, v_scale: float = 1.0, sliding_window: int = 0,
                      sinks=None, gate=None, out=None, q_rope: bool = False,
                      q_rope_theta: float = 10000.0, q_rope_offset: int = 0,
                      q_rope_dim: int = 0, split_tokens: int = 0, workspace=None,
                      v_tq_bits: int = 0, sparse_v_threshold: float = 0.0):
    """One-query-token paged decode attention (pkv_paged_decode_attn).

    q [S, Hq, Dqk]; k_cache [nb, B, Hkv, Dqk]; v_cache [nb, B, Hkv, Dv];
    block_tables int32 [S, M]; seq_lens int32 [S]; sinks FP32 [Hq] or None;
    gate FP32 [S, Hq, Dv] or None.  Returns out FP32 [S, Hq, Dv].
    ``workspace`` (uint8 device tensor) is allocated here when not given.
    ``sparse_v_threshold`` in [0, 1) (TQ V only): the sparse-V skip.
    """
    _dev(workspace)
    args, out, (S, Hq, Hkv, Dv, M, B) = _decode_args(
        q, k_cache, v_cache, block_tables, seq_lens, scale=scale, k_scale=k_scale,
        v_scale=v_scale, sparse_v_threshold=sparse_v_threshold, sliding_window=sliding_window,
        sinks=sinks, gate=gate, out=out, q_rope=q_rope, q_rope_theta=q_rope_theta,
        q_rope_offset=q_rope_offset, q_rope_dim=q_rope_dim, split_tokens=split_tokens,
        v_tq_bits=v_tq_bits, alloc_out=True)
    need = decode_workspace_bytes(S, Hq, Hkv, Dv, M, B, split_tokens, sliding_window) if S else 0
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().pkv_paged_decode_attn(*args, _ptr(workspace), ws_bytes, _stream()))
    return out


def paged_decode_attn_noalloc(q, k_cache, v_cache, block_tables, seq_lens, *, out,
                              scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                              sliding_window: int = 0, sinks=None, gate=None,
                              q_rope: bool = False, q_rope_theta: float = 10000.0,
                              q_rope_offset: int = 0, q_rope_dim: int = 0,
                              split_tokens: int = 0, v_tq_bits: int = 0,
                              sparse_v_threshold: float = 0.0):
    """paged_decode_attn with the split partials in the library's device
    scratch (pkv_paged_decode_attn_noalloc): allocates nothing, so ``out``
    must be given.  Calls that may overlap on one GPU share the scratch and
    race; at most PKV_DECODE_SCRATCH_BYTES (32 MiB) of partials."""
    args, out, _ = _decode_args(
        q, k_cache, v_cache, block_tables, seq_lens, scale=scale, k_scale=k_scale,
        v_scale=v_scale, sparse_v_threshold=sparse_v_threshold, sliding_window=sliding_window,
        sinks=sinks, gate=gate, out=out, q_rope=q_rope, q_rope_theta=q_rope_theta,
        q_rope_offset=q_rope_offset, q_rope_dim=q_rope_dim, split_tokens=split_tokens,
        v_tq_bits=v_tq_bits, alloc_out=False)
    _check(load().pkv_paged_decode_attn_noalloc(*args, _stream()))
    return out


def paged_prefill_attn(q, cu_q, k_cache, v_cache, block_tables, seq_lens, *, max_q_len: int,
                       scale: float, k_scale: float = 1.0, v_scale: float = 1.0,
                       sliding_window: int = 0, sinks=None, out=None):
    """Causal attention of the last q_len tokens of every sequence over the
    paged cache (pkv_paged_prefill_attn).

    q [total_q, Hq, D] BF16 (token stride free, heads packed); cu_q int32
    [S+1]; k_cache / v_cache [nb, B, Hkv, D]; block_tables int32 [S, M];
    seq_lens int32 [S] (including the new tokens); ``max_q_len`` >= every
    q_len (host value).  Returns out FP32 [total_q, Hq, D].
    """
    _dev(q, cu_q, k_cache, v_cache, block_tables, seq_lens, sinks, out)
    nb, B, Hkv, Dqk = _pool(k_cache, "k_cache")
    nb2, B2, Hkv2, Dv = _pool(v_cache, "v_cache")
    if (nb2, B2, Hkv2) != (nb, B, Hkv):
        raise ValueError("K and V pools must have the same blocks and heads")
    stride = _token_stride(q, "q")
    T, Hq = q.shape[0], q.shape[1]
    S = seq_lens.numel()
    if cu_q.dtype != torch.int32 or cu_q.numel() != S + 1 or not cu_q.is_contiguous():
        raise ValueError("cu_q must be int32 [S+1] contiguous")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or \
            block_tables.shape[0] != S or not block_tables.is_contiguous():
        raise ValueError("block_tables must be int32 [S, M] contiguous")
    if seq_lens.dtype != torch.int32 or not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be int32 [S] contiguous")
    if sinks is not None and (sinks.dtype != torch.float32 or sinks.numel() != Hq or
                              not sinks.is_contiguous()):
        raise ValueError("sinks must be FP32 [Hq] contiguous")
    if out is None:
        out = torch.zeros((T, Hq, Dv), dtype=torch.float32, device=q.device)
    elif out.dtype != torch.float32 or out.shape != (T, Hq, Dv) or not out.is_contiguous():
        raise ValueError("out must be FP32 [total_q, Hq, Dv] contiguous")
    _check(load().pkv_paged_prefill_attn(
        _ptr(q), _dtype(q), stride, _ptr(cu_q), max_q_len, T, _ptr(k_cache), _dtype(k_cache),
        k_scale, _ptr(v_cache), _dtype(v_cache), v_scale, _ptr(block_tables),
        block_tables.shape[1], _ptr(seq_lens), S, nb, Hq, Hkv, Dqk, Dv, B, scale, sliding_window,
        _ptr(sinks), _ptr(out), _stream()))
    return out


def mla_cache_assemble(kv_latent, k_rope, slot_mapping, k_cache, v_cache, *, kv_lora: int,
                       rope: int):
    """MLA cache rows at their slots (pkv_mla_cache_assemble): K = [latent |
    k_rope | 0], V = [latent | 0].  kv_latent [T, >= kv_lora] and k_rope
    [T, >= rope] (row stride free); caches [nb, B, 1, cache_dim]."""
    _dev(kv_latent, k_rope, slot_mapping, k_cache, v_cache)
    nb, B, H, dim = _pool(k_cache, "k_cache")
    if tuple(v_cache.shape) != (nb, B, H, dim) or not v_cache.is_contiguous() or H != 1:
        raise ValueError("caches must be [num_blocks, block_size, 1, cache_dim], alike")
    if kv_latent.dim() != 2 or kv_latent.stride(1) != 1 or k_rope.dim() != 2 or \
            k_rope.stride(1) != 1:
        raise ValueError("kv_latent and k_rope must be [T, width] with unit element stride")
    T = kv_latent.shape[0]
    if k_rope.shape[0] != T or slot_mapping.numel() != T or slot_mapping.dtype != torch.int64:
        raise ValueError("k_rope [T, rope] and slot_mapping int64 [T] must match kv_latent")
    dt = _dtype(kv_latent)
    if _dtype(k_rope) != dt or _dtype(k_cache) != dt or _dtype(v_cache) != dt:
        raise ValueError("kv_latent, k_rope and the caches must share one dtype")
    ls = kv_latent.stride(0) if T > 1 else kv_latent.shape[1]
    rs = k_rope.stride(0) if T > 1 else k_rope.shape[1]
    _check(load().pkv_mla_cache_assemble(
        _ptr(kv_latent), _ptr(k_rope), dt, ls, rs, _ptr(slot_mapping), T, kv_lora, rope, dim, B, nb,
        _ptr(k_cache), _ptr(v_cache), _stream()))
    return k_cache, v_cache
