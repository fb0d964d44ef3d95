"""Child process of tests/test_gpu_launch_contract.py, run under rocprofv3
with HIP API, kernel-dispatch, memory-copy and marker tracing.

Two roctx ranges around library calls whose inputs are already on the
device: "pkv_zero_work" holds every call with no work (zero tokens, zero
sequences), which must launch nothing (page 1, kv_cache.rs: the slot fill
returns before any launch when the count is 0); "pkv_calls" holds one call
of every entry point with work, which must launch only the library's kernels
and issue no memory copy, memset, allocation or synchronisation (the decode
state stays on the device; page 3, mla_cuda.rs: the device-resident KV
contract copies only the output back).  Prints the number of calls made."""
import ctypes
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import paged_kv_cache_fill_amd as pkv  # noqa: E402

roctx = ctypes.CDLL(os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib",
                                 "librocprofiler-sdk-roctx.so"))
roctx.roctxRangePushA.argtypes = [ctypes.c_char_p]


def main():
    dev = torch.device("cuda")
    pkv.load()
    H, Hq, D, B, S, n = 8, 32, 128, 16, 4, 300
    nblk = (n + B - 1) // B
    nb = S * nblk + 1
    bt = torch.arange(S * nblk, dtype=torch.int32, device=dev).view(S, nblk)
    lens = torch.full((S,), n, dtype=torch.int32, device=dev)
    kc = torch.zeros((nb, B, H, D), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    kc8 = torch.zeros((nb, B, H, D), dtype=torch.float8_e4m3fn, device=dev)
    vtq = torch.zeros((nb, pkv.v_block_bytes(pkv.TQ3, B, H, D)), dtype=torch.uint8, device=dev)
    T = S * n
    k_in = torch.randn((T, H, D), device=dev).to(torch.bfloat16)
    v_in = torch.randn((T, H, D), device=dev).to(torch.bfloat16)
    w = torch.ones(D, dtype=torch.bfloat16, device=dev)
    slots = torch.empty(T, dtype=torch.int64, device=dev)
    start = torch.zeros(S, dtype=torch.int32, device=dev)
    cu = torch.arange(0, T + 1, n, dtype=torch.int32, device=dev)
    pos = torch.arange(n, dtype=torch.int32, device=dev).repeat(S)
    q = torch.randn((S, Hq, D), device=dev).to(torch.bfloat16)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(pkv.decode_workspace_bytes(S, Hq, H, D, nblk, B) + 16, dtype=torch.uint8,
                     device=dev)
    qp = torch.randn((S * 32, Hq, D), device=dev).to(torch.bfloat16)
    cu_q = torch.arange(0, S * 32 + 1, 32, dtype=torch.int32, device=dev)
    outp = torch.empty((S * 32, Hq, D), dtype=torch.float32, device=dev)
    lat = torch.randn((T, 512), device=dev).to(torch.bfloat16)
    rope = torch.randn((T, 64), device=dev).to(torch.bfloat16)
    mk = torch.zeros((nb, B, 1, 576), dtype=torch.bfloat16, device=dev)
    mv = torch.zeros_like(mk)
    def calls():
        pkv.fill_slots(slots, bt, start, cu, B)
        pkv.cache_write_k_fused(k_in, slots, kc, norm_weight=w, pos_t=pos)
        pkv.cache_write_k_fused(k_in, slots, kc8, norm_weight=w, pos_t=pos, k_scale=0.5)
        pkv.cache_write_v(v_in, slots, vc)
        pkv.cache_write_v(v_in, slots, vtq, tq_bits=3)
        pkv.paged_decode_attn(q, kc, vc, bt, lens, scale=0.1, out=out, workspace=ws)
        pkv.paged_decode_attn(q, kc8, vtq, bt, lens, scale=0.1, k_scale=0.5, out=out,
                              workspace=ws, v_tq_bits=3)
        pkv.paged_decode_attn(q, kc8, vtq, bt, lens, scale=0.1, k_scale=0.5, out=out,
                              workspace=ws, v_tq_bits=3, sparse_v_threshold=0.01)
        pkv.paged_decode_attn_noalloc(q, kc, vc, bt, lens, scale=0.1, out=out)
        pkv.paged_prefill_attn(qp, cu_q, kc, vc, bt, lens, max_q_len=32, scale=0.1, out=outp)
        pkv.mla_cache_assemble(lat, rope, slots, mk, mv, kv_lora=512, rope=64)

    # empty inputs of the zero-work calls
    e_slots = torch.empty(0, dtype=torch.int64, device=dev)
    e_k = torch.empty((0, H, D), dtype=torch.bfloat16, device=dev)
    e_q = torch.empty((0, Hq, D), dtype=torch.bfloat16, device=dev)
    e_bt = torch.empty((0, nblk), dtype=torch.int32, device=dev)
    e_i32 = torch.empty(0, dtype=torch.int32, device=dev)
    e_out = torch.empty((0, Hq, D), dtype=torch.float32, device=dev)
    e_cu = torch.zeros(1, dtype=torch.int32, device=dev)
    e_lat = torch.empty((0, 512), dtype=torch.bfloat16, device=dev)
    e_rope = torch.empty((0, 64), dtype=torch.bfloat16, device=dev)
    e_outp = torch.empty((0, Hq, D), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    # every kernel launched once before the traced ranges (loading its code
    # object is the runtime's first-launch work, not the call's)
    calls()
    torch.cuda.synchronize()

    roctx.roctxRangePushA(b"pkv_zero_work")
    pkv.fill_slots(e_slots, e_bt, e_i32, e_cu, B)
    pkv.cache_write_k_fused(e_k, e_slots, kc, norm_weight=w, pos_t=e_i32)
    pkv.cache_write_k_fused(e_k, e_slots, kc8, norm_weight=w, pos_t=e_i32, k_scale=0.5)
    pkv.cache_write_v(e_k, e_slots, vc)
    pkv.cache_write_v(e_k, e_slots, vtq, tq_bits=3)
    pkv.paged_decode_attn(e_q, kc, vc, e_bt, e_i32, scale=0.1, out=e_out, workspace=ws)
    pkv.paged_decode_attn(e_q, kc8, vtq, e_bt, e_i32, scale=0.1, k_scale=0.5, out=e_out,
                          workspace=ws, v_tq_bits=3, sparse_v_threshold=0.01)
    pkv.paged_decode_attn_noalloc(e_q, kc, vc, e_bt, e_i32, scale=0.1, out=e_out)
    pkv.paged_prefill_attn(e_q, e_cu, kc, vc, e_bt, e_i32, max_q_len=1, scale=0.1, out=e_outp)
    pkv.mla_cache_assemble(e_lat, e_rope, e_slots, mk, mv, kv_lora=512, rope=64)
    roctx.roctxRangePop()
    torch.cuda.synchronize()

    roctx.roctxRangePushA(b"pkv_calls")
    calls()
    roctx.roctxRangePop()
    torch.cuda.synchronize()
    print("launch contract child: 10 zero-work calls, 11 calls with work", flush=True)


if __name__ == "__main__":
    main()
