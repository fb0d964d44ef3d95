"""The decode step (slot fill, fused K write, V write, decode attention with
its split-K merge) captured in a HIP graph and replayed: every replay, with
the program's own eager work and synchronisations in between, gives the
eager step's output and pools bit for bit.  Cases: BF16 V, 3-bit TQ V, and
3-bit TQ V with the sparse-V skip at a threshold (0.05) that both skips and
keeps blocks of these scores."""
import numpy as np
import pytest
import torch

import paged_kv_cache_fill_amd as pkv
import pkv_workloads as W
from _util import host, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("v_kind", ["bf16", "tq3", "tq3_sparse"])
def test_decode_step_graph_replays_match_eager(v_kind):
    lay = W.layout(2, num_seqs=32)
    cfg = lay.cfg
    S, Hq, Hkv, D, B = lay.num_seqs, cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], 16
    dev = torch.device("cuda")
    tq = 3 if v_kind.startswith("tq3") else 0
    tau = 0.05 if v_kind == "tq3_sparse" else 0.0
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    k_pool = torch.randn((lay.num_blocks, B, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    if tq:
        v_pool = torch.randint(0, 0x50, (lay.num_blocks, pkv.v_block_bytes(tq + 1, B, Hkv, D)),
                               dtype=torch.uint8, device=dev, generator=g)
    else:
        v_pool = torch.randn((lay.num_blocks, B, Hkv, D), device=dev, generator=g).to(torch.bfloat16)
    bt = torch.from_numpy(lay.block_tables).to(dev)
    seq_lens = torch.from_numpy(lay.seq_lens).to(dev)
    w = torch.from_numpy(W.norm_weight(2).view(np.int16)).to(dev).view(torch.bfloat16)
    k_new = W.device_normal(2, W.S_KNEW, (S, Hkv, D), torch.bfloat16, dev)
    v_new = W.device_normal(2, W.S_VNEW, (S, Hkv, D), torch.bfloat16, dev)
    q = W.device_normal(2, W.S_Q, (S, Hq, D), torch.bfloat16, dev)
    start, cu, pos = W.positions_decode(lay)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    start_t, cu_t, pos_t = i32(start), i32(cu), i32(pos)
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    out = torch.empty((S, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, pkv.decode_workspace_bytes(S, Hq, Hkv, D, lay.max_blocks_per_seq, B)),
                     dtype=torch.uint8, device=dev)

    def step():
        pkv.fill_slots(slots, bt, start_t, cu_t, B)
        pkv.cache_write_k_fused(k_new, slots, k_pool, norm_weight=w, eps=cfg["eps"], pos_t=pos_t,
                                theta=cfg["theta"])
        pkv.cache_write_v(v_new, slots, v_pool, tq_bits=tq)
        pkv.paged_decode_attn(q, k_pool, v_pool, bt, seq_lens, scale=D ** -0.5, out=out,
                              workspace=ws, v_tq_bits=tq, sparse_v_threshold=tau)

    say(f"graph replay of a decode step, V {v_kind}")
    step()
    torch.cuda.synchronize()
    ref = (host(out).copy(), host(k_pool).copy(), host(v_pool).copy(), host(slots).copy())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        out.fill_(float("nan"))                  # eager work between replays
        slots.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = (host(out), host(k_pool), host(v_pool), host(slots))
        for a, b, name in zip(got, ref, ("out", "k_pool", "v_pool", "slots")):
            assert a.tobytes() == b.tobytes(), f"replay {rep}: {name} differs"
