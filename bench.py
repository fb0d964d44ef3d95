"""Benchmark of the paged KV-cache hot path on one MI355X.

A step is one decode step of the whole path over a full-size batch:
  fill_slots (one new token per sequence, position seq_len-1)
  -> fused K write (RMSNorm, RoPE, one rounding) -> V write
  -> paged decode attention over every sequence's whole history.
The step is timed twice, as eager launches and as a replay of the step
captured once in a HIP graph (the same five launches); the faster of the two
is the step time and both are reported (--no-graph: eager launches only).
Before timing, the history of every sequence is written into the shuffled
pools through the same write calls (the population write); that write is
timed on its own and reported as the cache-write throughput.

Workloads (seeded, synthetic): ``decode_bf16_256seq`` (default; 256 sequences,
lengths U[512, 8192], Hq 32 / Hkv 8, D 128, BF16 K and V) and
``decode_fp8k_64seq_long`` (64 sequences, U[16384, 32768], Hq 64 / Hkv 8,
FP8 E4M3 K with k_scale = max|stored K| / 448, BF16 V).  Variants of the
latter: ``decode_fp8kv_64seq_long`` (E4M3 V too, v_scale = max|V| / 448) and
``decode_fp8k_64seq_long_window4096_sinks`` (a 4096-token sliding window and
one sink logit per query head; only the window's tokens are read and
counted).  ``write_prefill_16seq`` and ``decode_mla_gated_f32_4096`` are reported
workloads without a bar (the 16-sequence prefill cache write, scalar RoPE and
MRoPE; the one-sequence gated MLA-style FP32 decode, RoPE and NoPE), each call
timed after a scratch write that flushes the last-level cache.
``decode_bf16k_tq3v_256seq`` is the first workload with its V
cache in the 3-bit TurboQuant-style format (3-bit codes plus one E4M3 scale
per 16 elements: 0.4375 bytes per element); ``..._sparse_v`` is the same
with peaked attention (one heavy key every 64 positions, see SPARSE_V) and
the sparse-V skip at threshold 1e-3.  ``prefill_bf16_256seq_chunk256`` is chunked prefill on the first
workload's pool: the last min(256, n) tokens of every sequence are the new
chunk (slots, K write, V write, then causal prefill attention over the whole
cache); its metric is the attention's algorithmic TFLOP/s and its roofline
is the dense BF16 MFMA peak.

Prints one JSON line.  ``value`` is the algorithmic HBM bytes of one step
divided by the step time (GB/s); the decode attention's KV read is >99.9% of
those bytes.  ``roofline`` covers the decode attention call (its split-K
kernel and its merge kernel), timed with HIP events on the launch stream.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# name -> (workload index, V cache format, sliding window, sinks)
WORKLOADS = {
    "decode_bf16_256seq": (2, "bf16", 0, False),
    "decode_fp8k_64seq_long": (3, "bf16", 0, False),
    "decode_fp8kv_64seq_long": (3, "fp8", 0, False),
    "decode_fp8k_64seq_long_window4096_sinks": (3, "bf16", 4096, True),
    "decode_bf16k_tq3v_256seq": (2, "tq3", 0, False),
    "decode_bf16k_tq3v_256seq_sparse_v": (2, "tq3", 0, False),
}
# sparse-V workloads: name -> (threshold, heavy-position stride, heavy key
# length).  The history's key at every stride-th position (0, stride, ...)
# is replaced by heavy_len times the unit vector of the sum of its GQA
# group's queries, so that a few positions hold nearly all of the softmax
# mass (scores ~13-21 above the N(0, 1) bulk); the decode runs with the
# sparse-V skip at the threshold.
SPARSE_V = {"decode_bf16k_tq3v_256seq_sparse_v": (1e-3, 64, 40.0)}


def v_elem_bytes(v_kind):
    """Bytes per V element: 2 (BF16), 1 (E4M3), b/8 + 1/16 (b-bit TQ codes
    plus one E4M3 scale per 16 elements)."""
    if v_kind.startswith("tq"):
        return int(v_kind[2]) / 8 + 1 / 16
    return 1 if v_kind == "fp8" else 2
PREFILL_WORKLOADS = {"prefill_bf16_256seq_chunk256": (2, 256)}
# reported workloads with no bar: the 16-sequence prefill cache write (scalar
# RoPE and MRoPE with equal positions) and the one-sequence gated MLA-style
# FP32 decode (RoPE and NoPE); both fit in the 256 MB last-level cache, so
# every timed call follows a 512 MB scratch write that flushes it
AUX_WORKLOADS = {"write_prefill_16seq": 1, "decode_mla_gated_f32_4096": 4}
MFMA_BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="decode_bf16_256seq",
                   choices=sorted(WORKLOADS) + sorted(PREFILL_WORKLOADS) + sorted(AUX_WORKLOADS))
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--only", action="store_true",
                   help="with the default workload, leave out the second bar configuration "
                        "(decode_fp8k_64seq_long), which is otherwise run after it and "
                        "reported in the same line")
    p.add_argument("--split-tokens", type=int, default=0)
    p.add_argument("--no-graph", action="store_true",
                   help="time the decode step as eager launches only (by default also as a "
                        "HIP graph replay, and the faster of the two is the step time)")
    p.add_argument("--copy-probe", action="store_true",
                   help="only run a plain 2 GiB device copy (counter calibration)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# algorithmic bytes (what the method must move)
# --------------------------------------------------------------------------

def event_average(fn, reps, stream, rounds=3):
    """Average duration (ms) of one fn() call on `stream`, from HIP events
    recorded on that stream around a batch of `reps` back-to-back calls;
    the median of `rounds` batches, so that a batch in which the host or
    the device paused does not set the figure."""
    import torch
    res = []
    for _ in range(rounds):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        res.append(e0.elapsed_time(e1) / reps)
    return float(np.median(res))


def decode_bytes(lens, Hq, Hkv, D, Dv, kb, vb, qb, B=16, window=0, sinks=False):
    """KV rows read + block-table entries + seq_len + q read + FP32 out written
    (+ sink logits); with a window only the attended tokens [n - W, n) and the
    blocks that hold them count."""
    n = np.asarray(lens, np.int64)
    lo = np.where((window > 0) & (n > window), n - window, 0)
    kv = int(round(int((n - lo).sum()) * Hkv * (D * kb + Dv * vb)))
    bt = int(((n + B - 1) // B - lo // B).sum()) * 4
    S = n.size
    return (kv + bt + 4 * S + S * Hq * D * qb + S * Hq * Dv * 4
            + (Hq * 4 if sinks else 0))


def kwrite_bytes(T, Hkv, D, in_b, out_b):
    """K rows read and written, slot (8 B) and position (4 B) per token."""
    return T * (Hkv * D * (in_b + out_b) + 8 + 4)


def vwrite_bytes(T, Hkv, Dv, in_b, out_b):
    """V rows read and written, slot (8 B) per token."""
    return int(round(T * (Hkv * Dv * (in_b + out_b) + 8)))


def slots_bytes(T, S, B=16):
    return T * 8 + int(math.ceil(T / B)) * 4 + S * 8


# --------------------------------------------------------------------------

def copy_probe():
    import torch
    n = 2 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}))


def traffic_from_profile(kernel_src_hash: str, workload: str, kernel: str = "decode_attn",
                         suffix: str = "_pmc"):
    """HBM bytes per call measured with rocprofv3 --pmc (FETCH_SIZE and
    WRITE_SIZE, scaled by a plain copy's counters), stored in profiles/ with the
    hash of the kernel source they were taken on; None when stale or absent."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}{suffix}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_call:\s*([0-9.e+]+)", text)
    if not h or not t or h.group(1) != kernel_src_hash:
        return None
    return float(t.group(1))


def kernel_source_hash(source: str = "decode_attn.hip"):
    """Hash of a kernel's source file and the attention header it includes."""
    import hashlib
    h = hashlib.sha256()
    for name in (source, "attn_common.h"):
        h.update(open(os.path.join(ROOT, "paged_kv_cache_fill_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this path has no "
              "multi-GPU mode; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.copy_probe:
        copy_probe()
        return
    if args.workload in PREFILL_WORKLOADS:
        run_prefill(args)
        return
    if args.workload in AUX_WORKLOADS:
        run_aux(args)
        return

    result = run_decode(args.workload, args)
    if args.workload == "decode_bf16_256seq" and not args.only:
        # the second bar configuration in the same line: long-context decode
        # over an E4M3 K cache (64 sequences, U[16384, 32768])
        import torch
        torch.cuda.empty_cache()
        second = run_decode("decode_fp8k_64seq_long", args)
        result["decode_fp8k_64seq_long"] = {
            k: second[k] for k in ("config", "dtype", "value", "unit", "ms_per_step",
                                   "step_launch", "decode_attn", "cache_write", "roofline",
                                   "cpu_baseline")}
    print(json.dumps(result), flush=True)


def run_decode(name, args):
    """The decode-step benchmark of one workload; returns its result dict."""
    import torch

    import paged_kv_cache_fill_amd as pkv
    import pkv_workloads as W

    pkv.load()
    idx, v_kind, window, use_sinks = WORKLOADS[name]
    v_fp8 = v_kind == "fp8"
    tq = int(v_kind[2]) if v_kind.startswith("tq") else 0
    vb = v_elem_bytes(v_kind)
    lay = W.layout(idx)
    cfg = lay.cfg
    S, Hq, Hkv, D, B = lay.num_seqs, cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], 16
    Dv = cfg["head_dim_v"]
    fp8 = cfg["k_cache_dtype"] == "fp8"
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    log(f"workload {name}: {S} seqs, {lay.total_tokens} tokens, pool {lay.num_blocks} blocks")

    # ---------------- pools and the population write ----------------
    lens = lay.seq_lens.astype(np.int64)
    hist_lens = lens - 1
    Th = int(hist_lens.sum())
    kdt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    k_pool = torch.empty((lay.num_blocks, B, Hkv, D), dtype=kdt, device=dev)
    if tq:
        v_pool = torch.empty((lay.num_blocks, pkv.v_block_bytes(tq + 1, B, Hkv, Dv)),
                             dtype=torch.uint8, device=dev)
    else:
        vdt = torch.float8_e4m3fn if v_fp8 else torch.bfloat16
        v_pool = torch.empty((lay.num_blocks, B, Hkv, Dv), dtype=vdt, device=dev)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    w = torch.from_numpy(W.norm_weight(idx).view(np.int16)).to(dev).view(torch.bfloat16)

    k_hist = W.device_normal(idx, W.S_K, (Th, Hkv, D), torch.bfloat16, dev, outliers=fp8)
    v_hist = W.device_normal(idx, W.S_V, (Th, Hkv, Dv), torch.bfloat16, dev)
    start_h, cu_h, pos_h = W.positions_history(lay)
    slots_h = torch.empty(Th, dtype=torch.int64, device=dev)
    pos_h_t = torch.from_numpy(pos_h).to(dev)
    pkv.fill_slots(slots_h, bt, torch.from_numpy(start_h).to(dev),
                   torch.from_numpy(cu_h.astype(np.int32)).to(dev), B)

    k_scale = 1.0
    if fp8:
        k_scale = history_k_scale(k_hist, pos_h_t, w, cfg)
        log(f"k_scale = {k_scale:.6g}")
    v_scale = 1.0
    if v_fp8:
        v_scale = float(v_hist.abs().max().float().item()) / 448.0
        log(f"v_scale = {v_scale:.6g}")
    sinks = (torch.from_numpy(W.normal(idx, W.S_SINKS, (Hq,))).to(dev) if use_sinks else None)

    def populate():
        pkv.cache_write_k_fused(k_hist, slots_h, k_pool, norm_weight=w, eps=cfg["eps"],
                                pos_t=pos_h_t, theta=cfg["theta"], k_scale=k_scale)

    def populate_v():
        pkv.cache_write_v(v_hist, slots_h, v_pool, v_scale=v_scale, tq_bits=tq)

    def time_call(fn, reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for e0, e1 in evs:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    populate()
    populate_v()
    torch.cuda.synchronize()
    kw_ms = float(np.median(time_call(populate, 5)))
    vw_ms = float(np.median(time_call(populate_v, 5)))
    del k_hist, v_hist
    torch.cuda.empty_cache()
    kw_bytes = kwrite_bytes(Th, Hkv, D, 2, 1 if fp8 else 2)
    vw_bytes = vwrite_bytes(Th, Hkv, Dv, 2, vb)
    log(f"population write: K {kw_ms:.3f} ms ({kw_bytes / kw_ms / 1e6:.0f} GB/s), "
        f"V {vw_ms:.3f} ms ({vw_bytes / vw_ms / 1e6:.0f} GB/s)")

    # ---------------- the decode step ----------------
    k_new = W.device_normal(idx, W.S_KNEW, (S, Hkv, D), torch.bfloat16, dev, outliers=fp8)
    v_new = W.device_normal(idx, W.S_VNEW, (S, Hkv, Dv), torch.bfloat16, dev)
    q = W.device_normal(idx, W.S_Q, (S, Hq, D), torch.bfloat16, dev, outliers=fp8)
    spv_tau = 0.0
    if name in SPARSE_V:
        spv_tau, stride, heavy_len = SPARSE_V[name]
        n_heavy = heavy_keys(k_pool, q, lay, stride, heavy_len)
        log(f"sparse V: threshold {spv_tau:g}, {n_heavy} heavy keys (every {stride} positions)")
    start_d, cu_d, pos_d = W.positions_decode(lay)
    start_d_t = torch.from_numpy(start_d).to(dev)
    cu_d_t = torch.from_numpy(cu_d.astype(np.int32)).to(dev)
    pos_d_t = torch.from_numpy(pos_d).to(dev)
    slots_d = torch.empty(S, dtype=torch.int64, device=dev)
    out = torch.empty((S, Hq, Dv), dtype=torch.float32, device=dev)
    ws_n = pkv.decode_workspace_bytes(S, Hq, Hkv, Dv, lay.max_blocks_per_seq, B, args.split_tokens,
                                      window)
    ws = torch.empty(max(ws_n, 16), dtype=torch.uint8, device=dev)
    scale = D ** -0.5

    def step_writes():
        pkv.fill_slots(slots_d, bt, start_d_t, cu_d_t, B)
        pkv.cache_write_k_fused(k_new, slots_d, k_pool, norm_weight=w, eps=cfg["eps"],
                                pos_t=pos_d_t, theta=cfg["theta"], k_scale=k_scale)
        pkv.cache_write_v(v_new, slots_d, v_pool, v_scale=v_scale, tq_bits=tq)

    def step_attn():
        pkv.paged_decode_attn(q, k_pool, v_pool, bt, seq_lens, scale=scale, k_scale=k_scale,
                              v_scale=v_scale, sliding_window=window, sinks=sinks, out=out,
                              split_tokens=args.split_tokens, workspace=ws, v_tq_bits=tq,
                              sparse_v_threshold=spv_tau)

    def step():
        step_writes()
        step_attn()

    def timed(fn, k):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(k):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / k

    for _ in range(args.warmup):
        step()
    ms_eager = timed(step, args.steps)
    ms_graph = None
    if not args.no_graph:
        # the step's five launches captured once and replayed (same work, the
        # launches issued by the graph instead of the host)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        ms_graph = timed(graph.replay, args.steps)
    # the step is timed both ways (K steps each, synchronised on both sides);
    # the faster launch form is the step time, and both are reported
    use_graph = ms_graph is not None and ms_graph < ms_eager
    ms_per_step = ms_graph if use_graph else ms_eager

    # average call durations from HIP events on the launch stream (median of three batches)
    attn_ms = event_average(step_attn, args.steps, stream)
    write_ms = event_average(step_writes, args.steps, stream)
    log(f"step {ms_per_step:.3f} ms ({'graph replay' if use_graph else 'eager'}; eager "
        f"{ms_eager:.3f} ms, graph {'-' if ms_graph is None else f'{ms_graph:.3f}'} ms; decode call "
        f"{attn_ms:.3f} ms, step writes {write_ms * 1e3:.1f} us)")

    dec_b = decode_bytes(lens, Hq, Hkv, D, Dv, 1 if fp8 else 2, vb, 2,
                         window=window, sinks=use_sinks)
    step_b = (dec_b + kwrite_bytes(S, Hkv, D, 2, 1 if fp8 else 2)
              + vwrite_bytes(S, Hkv, Dv, 2, vb) + slots_bytes(S, S))
    value = step_b / (ms_per_step * 1e-3) / 1e9
    achieved = dec_b / (attn_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(kernel_source_hash(), name)

    result = {
        "metric": "paged decode-attn KV GB/s + cache-write tokens/s (fraction of HBM peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_step_eager": round(ms_eager, 4),
        "ms_per_step_graph": None if ms_graph is None else round(ms_graph, 4),
        "step_launch": "hip_graph" if use_graph else "eager",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": (("fp8_e4m3 K" if fp8 else "bf16 K")
                  + {"fp8": " / fp8_e4m3 V", "bf16": " / bf16 V"}.get(
                      v_kind, f" / {tq}-bit TQ V (e4m3 scale per 16)")
                  + ", f32 accumulate"),
        "data": "synthetic (seeded)",
        "config": {"workload": name, "num_seqs": S, "seq_len_range": [cfg["len_lo"], cfg["len_hi"]],
                   "total_tokens": int(lens.sum()), "num_q_heads": Hq, "num_kv_heads": Hkv,
                   "head_dim": D, "block_size": B, "sliding_window": window,
                   "sinks": use_sinks, "parallelism": "single GPU"},
        "decode_attn": {"ms": round(attn_ms, 4), "algorithmic_bytes": dec_b,
                        "GB_per_s": round(achieved, 1), "frac_of_hbm_peak": round(achieved / HBM_PEAK_GBS, 4)},
        "cache_write": {
            "population_tokens": Th,
            "k_fused": {"ms": round(kw_ms, 4), "tokens_per_s": round(Th / kw_ms * 1e3),
                        "GB_per_s": round(kw_bytes / kw_ms / 1e6, 1),
                        "frac_of_hbm_peak": round(kw_bytes / kw_ms / 1e6 / HBM_PEAK_GBS, 4)},
            "v": {"ms": round(vw_ms, 4), "tokens_per_s": round(Th / vw_ms * 1e3),
                  "GB_per_s": round(vw_bytes / vw_ms / 1e6, 1),
                  "frac_of_hbm_peak": round(vw_bytes / vw_ms / 1e6 / HBM_PEAK_GBS, 4)},
            "decode_step_writes_us": round(write_ms * 1e3, 2),
        },
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "paged_decode_attn (split-K + merge)"},
        "cpu_baseline": None,
    }
    if name in SPARSE_V:
        result["config"].update(sparse_v_threshold=spv_tau, heavy_key_stride=stride,
                                heavy_key_length=heavy_len)
        result["roofline"]["note"] = ("achieved counts the exact decode's algorithmic bytes; "
                                      "the V of skipped blocks is not read, so the measured "
                                      "traffic is below them")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(idx, lay, k_scale, v_kind, v_scale, window,
                                              None if sinks is None else sinks.cpu().numpy(),
                                              sparse_v=SPARSE_V.get(name))
    return result


def heavy_keys(k_pool, q, lay, stride, heavy_len):
    """Writes the heavy keys of a sparse-V workload into a BF16 K pool
    [nb, 16, Hkv, D]: at history positions 0, stride, 2 stride, ... of every
    sequence, for every kv head, heavy_len times the unit vector of the sum
    of the head's GQA group of queries q [S, Hq, D].  Returns their count."""
    import torch
    S, Hq, D = q.shape
    Hkv = k_pool.shape[2]
    u = q.float().view(S, Hkv, Hq // Hkv, D).sum(2)
    u = u / u.norm(dim=-1, keepdim=True)
    seq, pos = [], []
    for s in range(S):
        t = np.arange(0, int(lay.seq_lens[s]) - 1, stride)
        seq.append(np.full(t.size, s))
        pos.append(t)
    seq, pos = np.concatenate(seq), np.concatenate(pos)
    blk = lay.block_tables[seq, pos // 16]
    dev = k_pool.device
    k_pool[torch.from_numpy(blk).to(dev).long(), torch.from_numpy(pos % 16).to(dev).long()] = \
        (heavy_len * u[torch.from_numpy(seq).to(dev).long()]).to(k_pool.dtype)
    return int(seq.size)


def history_k_scale(k_hist, pos, w, cfg, B=16):
    """k_scale = max |stored FP32 K| / 448 over a history K [T, Hkv, D]: the K
    path's FP32 output (RMSNorm and RoPE through the library's FP32 store),
    computed in chunks."""
    import torch

    import paged_kv_cache_fill_amd as pkv
    T, Hkv, D = k_hist.shape
    dev = k_hist.device
    amax = torch.zeros((), dtype=torch.float32, device=dev)
    chunk = 1 << 16
    tmp = torch.empty((chunk // B, B, Hkv, D), dtype=torch.float32, device=dev)
    ident = torch.arange(chunk, dtype=torch.int64, device=dev)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        pkv.cache_write_k_fused(k_hist[t0:t1], ident[:t1 - t0], tmp, norm_weight=w,
                                eps=cfg["eps"], pos_t=pos[t0:t1], theta=cfg["theta"])
        amax = torch.maximum(amax, tmp.view(-1)[:(t1 - t0) * Hkv * D].abs().max())
    return float(amax.item()) / 448.0


def prefill_flops(lens, qlens, Hq, D, Dv):
    """Algorithmic FLOPs of causal prefill attention: query i of a sequence
    of n tokens with q_len new ones attends to n - q_len + i + 1 keys, each
    costing 2 D (q.k) + 2 Dv (p v) per query head."""
    keys = 0
    for n, c in zip(np.asarray(lens, np.int64), np.asarray(qlens, np.int64)):
        keys += int(c * (n - c) + c * (c + 1) // 2)
    return keys * Hq * (2 * D + 2 * Dv)


def run_prefill(args):
    import torch

    import paged_kv_cache_fill_amd as pkv
    import pkv_workloads as W

    pkv.load()
    idx, chunk = PREFILL_WORKLOADS[args.workload]
    lay = W.layout(idx)
    cfg = lay.cfg
    S, Hq, Hkv, D, B = lay.num_seqs, cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], 16
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    lens = lay.seq_lens.astype(np.int64)
    qlens = np.minimum(lens, chunk)
    hist = lens - qlens
    Th, Tc = int(hist.sum()), int(qlens.sum())
    log(f"workload {args.workload}: {S} seqs, {int(lens.sum())} tokens, chunk {chunk} "
        f"({Tc} new tokens), pool {lay.num_blocks} blocks")
    k_pool = torch.empty((lay.num_blocks, B, Hkv, D), dtype=torch.bfloat16, device=dev)
    v_pool = torch.empty_like(k_pool)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    w = torch.from_numpy(W.norm_weight(idx).view(np.int16)).to(dev).view(torch.bfloat16)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    def positions(start, count):
        cu = np.zeros(S + 1, np.int64)
        cu[1:] = np.cumsum(count)
        pos = np.concatenate([np.arange(a, a + c, dtype=np.int32) for a, c in zip(start, count)])
        return i32(start), i32(cu), i32(pos), int(cu[-1])

    # history: the first n - q_len tokens of every sequence, written once
    hs, hcu, hpos, _ = positions(np.zeros(S, np.int64), hist)
    k_hist = W.device_normal(idx, W.S_K, (Th, Hkv, D), torch.bfloat16, dev)
    v_hist = W.device_normal(idx, W.S_V, (Th, Hkv, D), torch.bfloat16, dev)
    slots_h = torch.empty(Th, dtype=torch.int64, device=dev)
    pkv.fill_slots(slots_h, bt, hs, hcu, B)
    pkv.cache_write_k_fused(k_hist, slots_h, k_pool, norm_weight=w, eps=cfg["eps"], pos_t=hpos,
                            theta=cfg["theta"])
    pkv.cache_write_v(v_hist, slots_h, v_pool)
    del k_hist, v_hist
    # the chunk: slots, K write, V write, prefill attention
    cs, ccu, cpos, _ = positions(hist, qlens)
    k_new = W.device_normal(idx, W.S_KNEW, (Tc, Hkv, D), torch.bfloat16, dev)
    v_new = W.device_normal(idx, W.S_VNEW, (Tc, Hkv, D), torch.bfloat16, dev)
    q = W.device_normal(idx, W.S_Q, (Tc, Hq, D), torch.bfloat16, dev)
    slots_c = torch.empty(Tc, dtype=torch.int64, device=dev)
    out = torch.empty((Tc, Hq, D), dtype=torch.float32, device=dev)
    scale = D ** -0.5

    def step_writes():
        pkv.fill_slots(slots_c, bt, cs, ccu, B)
        pkv.cache_write_k_fused(k_new, slots_c, k_pool, norm_weight=w, eps=cfg["eps"], pos_t=cpos,
                                theta=cfg["theta"])
        pkv.cache_write_v(v_new, slots_c, v_pool)

    def step_attn():
        pkv.paged_prefill_attn(q, ccu, k_pool, v_pool, bt, seq_lens, max_q_len=chunk,
                               scale=scale, out=out)

    def step():
        step_writes()
        step_attn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    attn_ms = event_average(step_attn, args.steps, stream)
    write_ms = event_average(step_writes, args.steps, stream)
    flops = prefill_flops(lens, qlens, Hq, D, D)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms (prefill attention {attn_ms:.3f} ms = {tflops:.1f} TFLOP/s, "
        f"chunk writes {write_ms * 1e3:.1f} us)")
    result = {
        "metric": "paged prefill attention TFLOP/s (chunked prefill over the paged cache)",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 q/K/V, f32 accumulate",
        "data": "synthetic (seeded)",
        "config": {"workload": args.workload, "num_seqs": S, "chunk": chunk,
                   "new_tokens": Tc, "total_tokens": int(lens.sum()), "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": B,
                   "parallelism": "single GPU"},
        "prefill_attn": {"ms": round(attn_ms, 4), "algorithmic_flops": flops,
                         "TFLOP_per_s": round(tflops, 1)},
        "chunk_writes_us": round(write_ms * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 1),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": traffic_from_profile(kernel_source_hash("prefill_attn.hip"),
                                                     args.workload, "prefill_attn"),
                     "kernel": "paged_prefill_attn"},
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


def run_aux(args):
    """The two reported workloads.  Each call is timed with HIP events on the
    launch stream after a 512 MB scratch write (outside the timed region) that
    flushes the last-level cache; the median of `steps` calls is reported."""
    import torch

    import oracle
    import paged_kv_cache_fill_amd as pkv
    import pkv_workloads as W

    pkv.load()
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    idx = AUX_WORKLOADS[args.workload]
    lay = W.layout(idx)
    cfg = lay.cfg
    Hkv, D, Dv, B = cfg["num_kv_heads"], cfg["head_dim"], cfg["head_dim_v"], 16
    bt = torch.from_numpy(lay.block_tables).to(dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        ts = []
        for _ in range(args.steps):
            flush.fill_(1)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)

    if idx == 1:
        start, cu, pos = W.positions_all(lay)
        T, S = int(cu[-1]), lay.num_seqs
        k_h, v_h, w_h = W.kv_tokens(1, T, "k"), W.kv_tokens(1, T, "v"), W.norm_weight(1)
        k = torch.from_numpy(k_h.view(np.int16)).to(dev).view(torch.bfloat16)
        v = torch.from_numpy(v_h.view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(w_h.view(np.int16)).to(dev).view(torch.bfloat16)
        k_pool = torch.empty((lay.num_blocks, B, Hkv, D), dtype=torch.bfloat16, device=dev)
        v_pool = torch.empty_like(k_pool)
        slots = torch.empty(T, dtype=torch.int64, device=dev)
        st, cut, post = i32(start), i32(cu), i32(pos)
        calls = {
            "fill_slots": (lambda: pkv.fill_slots(slots, bt, st, cut, B), slots_bytes(T, S)),
            "k_fused": (lambda: pkv.cache_write_k_fused(k, slots, k_pool, norm_weight=w,
                                                        eps=cfg["eps"], pos_t=post,
                                                        theta=cfg["theta"]),
                        kwrite_bytes(T, Hkv, D, 2, 2)),
            "k_fused_mrope": (lambda: pkv.cache_write_k_fused(k, slots, k_pool, norm_weight=w,
                                                              eps=cfg["eps"], pos_t=post,
                                                              pos_h=post, pos_w=post,
                                                              theta=cfg["theta"]),
                              kwrite_bytes(T, Hkv, D, 2, 2) + 8 * T),
            "v": (lambda: pkv.cache_write_v(v, slots, v_pool), vwrite_bytes(T, Hkv, D, 2, 2)),
        }
        res = {}
        for name, (fn, nb) in calls.items():
            ms = timed(fn)
            res[name] = {"ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3)),
                         "GB_per_s": round(nb / ms / 1e6, 1),
                         "frac_of_hbm_peak": round(nb / ms / 1e6 / HBM_PEAK_GBS, 4)}
            log(f"{name}: {ms * 1e3:.1f} us ({nb / ms / 1e6:.0f} GB/s)")
        step_ms = res["fill_slots"]["ms"] + res["k_fused"]["ms"] + res["v"]["ms"]
        step_b = slots_bytes(T, S) + kwrite_bytes(T, Hkv, D, 2, 2) + vwrite_bytes(T, Hkv, D, 2, 2)
        dom = "k_fused"
        dom_b = kwrite_bytes(T, Hkv, D, 2, 2)
        traffic = traffic_from_profile(kernel_source_hash("cache_write_k.hip"), args.workload,
                                       kernel="cache_write", suffix="")
        # the oracle on the same inputs: slots, K write, V write
        kc = np.zeros((lay.num_blocks, B, Hkv, D), np.uint16)
        vc = np.zeros_like(kc)

        def run(threads):
            t0 = time.perf_counter()
            s_ref = oracle.fill_slots(lay.block_tables, start, cu, T, B)
            oracle.cache_write_k(k_h, "bf16", s_ref, kc, "bf16", num_kv_heads=Hkv, head_dim=D,
                                 block_size=B, norm_weight=w_h, eps=cfg["eps"], pos_t=pos,
                                 theta=cfg["theta"], nthreads=threads)
            oracle.cache_write_v(v_h, "bf16", s_ref, vc, num_kv_heads=Hkv, head_dim_v=D,
                                 block_size=B)
            return time.perf_counter() - t0

        cpu = oracle_timing(run, step_b, f"slots, K write and V write of all {T} tokens")
        config = {"workload": args.workload, "num_seqs": S, "tokens": T, "num_kv_heads": Hkv,
                  "head_dim": D, "block_size": B, "pool_blocks": lay.num_blocks,
                  "parallelism": "single GPU"}
        dtype = "bf16 in / bf16 cache, f32 K path"
    else:
        H, n = cfg["num_q_heads"], int(lay.seq_lens[0])
        kp = W.device_normal(4, W.S_POOLK, (lay.num_blocks, B, Hkv, D), torch.float32, dev)
        vp = W.device_normal(4, W.S_POOLV, (lay.num_blocks, B, Hkv, Dv), torch.float32, dev)
        k_new = W.device_normal(4, W.S_KNEW, (1, Hkv, D), torch.float32, dev)
        v_new = W.device_normal(4, W.S_VNEW, (1, Hkv, Dv), torch.float32, dev)
        q_h, g_h = W.queries(4, 1), W.gate(4, 1)
        q, g = torch.from_numpy(q_h).to(dev), torch.from_numpy(g_h).to(dev)
        seq_lens = i32(lay.seq_lens)
        slot = torch.empty(1, dtype=torch.int64, device=dev)
        st, cut, post = i32([n - 1]), i32([0, 1]), i32([n - 1])
        out = torch.empty((1, H, Dv), dtype=torch.float32, device=dev)
        ws = torch.empty(max(16, pkv.decode_workspace_bytes(1, H, Hkv, Dv, lay.max_blocks_per_seq,
                                                            B, args.split_tokens)),
                         dtype=torch.uint8, device=dev)
        rope = dict(theta=cfg["theta"], rope_offset=cfg["rope_offset"],
                    rotary_dim=cfg["rotary_dim"])

        def step(nope):
            pkv.fill_slots(slot, bt, st, cut, B)
            pkv.cache_write_k_fused(k_new, slot, kp, pos_t=post, nope=nope, **rope)
            pkv.cache_write_v(v_new, slot, vp)
            pkv.paged_decode_attn(q, kp, vp, bt, seq_lens, scale=D ** -0.5, gate=g, out=out,
                                  q_rope=not nope, q_rope_theta=cfg["theta"],
                                  q_rope_offset=cfg["rope_offset"],
                                  q_rope_dim=cfg["rotary_dim"], workspace=ws,
                                  split_tokens=args.split_tokens)

        dec_b = decode_bytes(lay.seq_lens, H, Hkv, D, Dv, 4, 4, 4) + H * Dv * 4   # + gate
        res = {}
        for name, nope in (("rope", False), ("nope", True)):
            ms = timed(lambda: step(nope))
            res[name] = {"ms": round(ms, 4), "GB_per_s": round(dec_b / ms / 1e6, 1),
                         "frac_of_hbm_peak": round(dec_b / ms / 1e6 / HBM_PEAK_GBS, 4)}
            log(f"step ({name}): {ms * 1e3:.1f} us ({dec_b / ms / 1e6:.0f} GB/s)")
        dmsv = timed(lambda: pkv.paged_decode_attn(q, kp, vp, bt, seq_lens, scale=D ** -0.5,
                                                   gate=g, out=out, q_rope=True,
                                                   q_rope_theta=cfg["theta"],
                                                   q_rope_offset=cfg["rope_offset"],
                                                   q_rope_dim=cfg["rotary_dim"], workspace=ws,
                                                   split_tokens=args.split_tokens))
        res["decode_call"] = {"ms": round(dmsv, 4), "GB_per_s": round(dec_b / dmsv / 1e6, 1),
                              "frac_of_hbm_peak": round(dec_b / dmsv / 1e6 / HBM_PEAK_GBS, 4)}
        step_ms, step_b = res["rope"]["ms"], dec_b
        dom, dom_b = "decode_call", dec_b
        traffic = traffic_from_profile(kernel_source_hash(), args.workload)
        # the oracle: attention over the same pools (copied to the host)
        kp_h, vp_h = kp.cpu().numpy(), vp.cpu().numpy()

        def run(threads):
            t0 = time.perf_counter()
            oracle.paged_decode(q_h, "f32", kp_h, "f32", vp_h, "f32", lay.block_tables,
                                lay.seq_lens, num_q_heads=H, num_kv_heads=Hkv, head_dim_qk=D,
                                head_dim_v=Dv, block_size=B, scale=D ** -0.5, q_rope=True,
                                q_rope_theta=cfg["theta"], q_rope_offset=cfg["rope_offset"],
                                q_rope_dim=cfg["rotary_dim"], gate=g_h, nthreads=threads)
            return time.perf_counter() - t0

        cpu = oracle_timing(run, dec_b, f"gated decode attention over {n} tokens")
        config = {"workload": args.workload, "num_seqs": 1, "seq_len": n, "num_heads": H,
                  "head_dim_qk": D, "head_dim_v": Dv, "rope_dim": cfg["rotary_dim"],
                  "theta": cfg["theta"], "parallelism": "single GPU"}
        dtype = "f32"
    achieved = dom_b / (res[dom]["ms"] * 1e-3) / 1e9
    result = {
        "metric": "paged decode-attn KV GB/s + cache-write tokens/s (fraction of HBM peak)",
        "value": round(step_b / (step_ms * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded)",
        "config": config,
        "calls": res,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": dom},
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


# tokens of the bounded CPU sample per workload: the first sequences of the
# workload, in its order, until this many tokens (about 4 s of one-thread
# oracle work on a 2.7 GHz Xeon core; BF16 K costs ~28 us a token, E4M3 K
# with 64 query heads ~100 us)
CPU_SAMPLE_TOKENS = {2: 131072, 3: 40960}


def host_cpu():
    """CPU model, logical CPUs of the host, and the CPUs this process may
    use (its affinity mask)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return model, os.cpu_count() or 1, usable


def oracle_timing(run, nbytes, sample, unit_scale=1e9, unit="GB/s"):
    """Times run(threads) -- one pass of the oracle over a sample -- on one
    thread and on all threads this process may use (at most 16, the CPU
    share of one GPU on the benchmark hosts), median of 3 runs each; nbytes
    (or flops) / time in `unit`."""
    model, logical, usable = host_cpu()
    cores = max(1, min(16, usable))
    t1 = float(np.median([run(1) for _ in range(3)]))
    tn = float(np.median([run(cores) for _ in range(3)]))
    log(f"cpu baseline ({sample}): 1 thread {t1:.3f} s, {cores} threads {tn:.3f} s")
    return {"value": round(nbytes / tn / unit_scale, 4), "unit": unit, "cores": cores,
            "kind": "oracle", "value_1thread": round(nbytes / t1 / unit_scale, 4),
            "value_all": round(nbytes / tn / unit_scale, 4), "seconds_1thread": round(t1, 4),
            "seconds_all": round(tn, 4), "cpu_model": model, "host_logical_cpus": logical,
            "usable_cpus": usable, "sample": f"{sample}; median of 3 runs on 1 thread and on "
                                             f"{cores}"}


def cpu_baseline(idx, lay, k_scale, v_kind="bf16", v_scale=1.0, window=0, sinks=None,
                 sparse_v=None):
    """The oracle, as it stands, timed on this host on a bounded sample of the
    decode step: the first sequences of the workload (in its order) up to
    CPU_SAMPLE_TOKENS tokens -- slots, K write and V write of their new
    tokens, attention over their whole histories -- on one thread and on
    all the threads this process may use (at most 16, the CPU share of one
    GPU on the benchmark hosts), median of 3 runs each.  The sampled
    sequences' blocks are drawn by the seeded generator on the device and
    copied to the host; nothing in them comes from the HIP path.  With
    sparse_v = (threshold, stride, heavy length) the sample gets the heavy
    keys of the sparse-V workload and the oracle's sparse-V decode runs."""
    import torch

    import oracle
    import pkv_workloads as W
    cfg = lay.cfg
    Hq, Hkv, D, Dv = cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], cfg["head_dim_v"]
    fp8 = cfg["k_cache_dtype"] == "fp8"
    lens_all = lay.seq_lens.astype(np.int64)
    S = int(np.searchsorted(np.cumsum(lens_all), CPU_SAMPLE_TOKENS.get(idx, 1 << 17)) + 1)
    S = min(S, lay.num_seqs)
    lens = lay.seq_lens[:S].copy()
    nblk = (lens.astype(np.int64) + 15) // 16
    M = int(nblk.max())
    ids = np.unique(np.concatenate([lay.block_tables[s, :nblk[s]] for s in range(S)]))
    remap = np.zeros(lay.num_blocks, np.int32)
    remap[ids] = np.arange(ids.size, dtype=np.int32)
    bt = np.zeros((S, M), np.int32)
    for s in range(S):
        bt[s, :nblk[s]] = remap[lay.block_tables[s, :nblk[s]]]
    nb = int(ids.size)
    shape = (nb, 16, Hkv, D)
    vshape = (nb, 16, Hkv, Dv)

    def codes(stream, shp):
        g = torch.Generator(device="cuda")
        g.manual_seed(W.seed_of(idx) * 1000 + stream)
        mag = torch.randint(0, 0x50, shp, dtype=torch.uint8, device="cuda", generator=g)
        sign = torch.randint(0, 2, shp, dtype=torch.uint8, device="cuda", generator=g) << 7
        return (mag | sign).cpu().numpy()

    if fp8:
        kp = codes(W.S_POOLK, shape)
    else:
        kp = W.device_normal(idx, W.S_POOLK, shape, torch.bfloat16, "cuda").view(torch.int16) \
            .cpu().numpy().view(np.uint16)
    vb = v_elem_bytes(v_kind)
    if v_kind.startswith("tq"):
        # random code bytes and random finite E4M3 scales; a block is one
        # region per kv head: 16 code rows, then Dv / 16 scale rows of 16 bytes
        bits = int(v_kind[2])
        cb, sb = 16 * Dv * bits // 8, 16 * Dv // 16
        vp = np.concatenate([codes(W.S_POOLV, (nb, Hkv, cb)),
                             codes(W.S_POOLV + 1, (nb, Hkv, sb)) & 0x7F], axis=2).reshape(nb, -1)
    elif v_kind == "fp8":
        vp = codes(W.S_POOLV, vshape)
    else:
        vp = W.device_normal(idx, W.S_POOLV, vshape, torch.bfloat16, "cuda") \
            .view(torch.int16).cpu().numpy().view(np.uint16)
    torch.cuda.empty_cache()
    q = W.queries(idx, lay.num_seqs)[:S]
    k_new = W.kv_tokens(idx, lay.num_seqs, "k")[:S]
    v_new = W.kv_tokens(idx, lay.num_seqs, "v")[:S]
    w = W.norm_weight(idx)
    sub = W.Layout(idx, lens, bt, nb, -1, 16, cfg)
    start, cu, pos = W.positions_decode(sub)

    if sparse_v is not None:
        _, stride, heavy_len = sparse_v
        G = Hq // Hkv
        u = oracle.to_f64(q, "bf16").reshape(S, Hkv, G, D).sum(2)
        u /= np.linalg.norm(u, axis=-1, keepdims=True)
        for s in range(S):
            for t in range(0, int(lens[s]) - 1, stride):
                kp[bt[s, t // 16], t % 16] = W.bf16_bits((heavy_len * u[s]).astype(np.float32))

    def decode(threads):
        kw = dict(num_q_heads=Hq, num_kv_heads=Hkv, head_dim_qk=D, head_dim_v=Dv, block_size=16,
                  scale=D ** -0.5, k_scale=k_scale, v_scale=v_scale, sliding_window=window,
                  sinks=sinks, nthreads=threads)
        if sparse_v is not None:
            oracle.paged_decode_sparse_v(q, "bf16", kp, cfg["k_cache_dtype"], vp, v_kind, bt,
                                         lens, tau=sparse_v[0], **kw)
        else:
            oracle.paged_decode(q, "bf16", kp, cfg["k_cache_dtype"], vp, v_kind, bt, lens, **kw)

    def run(threads):
        t0 = time.perf_counter()
        slots = oracle.fill_slots(bt, start, cu, S, 16)
        oracle.cache_write_k(k_new, "bf16", slots, kp, cfg["k_cache_dtype"], num_kv_heads=Hkv,
                             head_dim=D, block_size=16, norm_weight=w, eps=cfg["eps"], pos_t=pos,
                             theta=cfg["theta"], k_scale=k_scale, nthreads=threads)
        oracle.cache_write_v(v_new, "bf16", slots, vp, num_kv_heads=Hkv, head_dim_v=Dv,
                             block_size=16, cache_dtype=v_kind, v_scale=v_scale)
        decode(threads)
        return time.perf_counter() - t0

    b = (decode_bytes(lens, Hq, Hkv, D, Dv, 1 if fp8 else 2, vb, 2, window=window,
                      sinks=sinks is not None)
         + kwrite_bytes(S, Hkv, D, 2, 1 if fp8 else 2)
         + vwrite_bytes(S, Hkv, Dv, 2, vb) + slots_bytes(S, S))
    what = "sparse-V attention" if sparse_v is not None else "attention"
    return oracle_timing(run, b, f"decode step (slots, K and V write of the new token, "
                                 f"{what} over the whole history) of the first {S} of "
                                 f"{lay.num_seqs} sequences, {int(lens.sum())} tokens")


if __name__ == "__main__":
    main()
