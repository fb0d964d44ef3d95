"""Host-side logic of bench.py, on the CPU: the one-GPU contract of the
command line, the algorithmic byte counts against counts made by hand, the
hash lock of the traffic figures taken from profiles/, and the heavy keys of
the sparse-V workload."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import bench
import pkv_workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_decode_bytes_by_hand():
    # two sequences of 17 and 32 tokens, Hq 4 / Hkv 2, D 8, BF16 K and V, BF16 q:
    # KV rows (17 + 32) * 2 * (8*2 + 8*2); table entries (2 + 2) * 4; seq_lens
    # 2 * 4; q 2 * 4 * 8 * 2; out 2 * 4 * 8 * 4
    want = 49 * 2 * 32 + 16 + 8 + 128 + 256
    assert bench.decode_bytes([17, 32], 4, 2, 8, 8, 2, 2, 2) == want
    # a window of 10: tokens [7, 17) and [22, 32); blocks 0-1 and 1-1
    want_w = 20 * 2 * 32 + (2 + 1) * 4 + 8 + 128 + 256
    assert bench.decode_bytes([17, 32], 4, 2, 8, 8, 2, 2, 2, window=10) == want_w
    # sinks add one FP32 logit per query head
    assert bench.decode_bytes([17], 4, 2, 8, 8, 2, 2, 2, sinks=True) == \
        bench.decode_bytes([17], 4, 2, 8, 8, 2, 2, 2) + 16


def test_element_bytes_of_the_v_formats():
    assert bench.v_elem_bytes("bf16") == 2
    assert bench.v_elem_bytes("fp8") == 1
    # b-bit codes plus one E4M3 scale per 16 elements
    assert bench.v_elem_bytes("tq2") == 0.25 + 1 / 16
    assert bench.v_elem_bytes("tq3") == 0.4375
    assert bench.v_elem_bytes("tq4") == 0.5625


def test_write_and_slot_bytes_by_hand():
    assert bench.kwrite_bytes(3, 2, 8, 2, 1) == 3 * (2 * 8 * 3 + 12)
    assert bench.vwrite_bytes(3, 2, 8, 2, 2) == 3 * (2 * 8 * 4 + 8)
    assert bench.slots_bytes(33, 2) == 33 * 8 + 3 * 4 + 16


def test_traffic_is_taken_only_for_the_hash_it_was_measured_on():
    h = bench.kernel_source_hash()
    got = bench.traffic_from_profile(h, "decode_bf16_256seq")
    assert got is not None and 4.4e9 < got < 4.6e9
    assert bench.traffic_from_profile("0" * 16, "decode_bf16_256seq") is None
    assert bench.traffic_from_profile(h, "no_such_workload") is None


def test_every_decode_workload_has_a_current_profile():
    h = bench.kernel_source_hash()
    for name in bench.WORKLOADS:
        assert bench.traffic_from_profile(h, name) is not None, name
    hp = bench.kernel_source_hash("prefill_attn.hip")
    for name in bench.PREFILL_WORKLOADS:
        assert bench.traffic_from_profile(hp, name, "prefill_attn") is not None, name


def test_heavy_keys_of_the_sparse_v_workload():
    lay = W.layout_for(2, [5, 40, 130])
    Hq, Hkv, D = 8, 2, 16
    pool = torch.zeros((lay.num_blocks, 16, Hkv, D), dtype=torch.bfloat16)
    q = torch.from_numpy(W.normal(2, 7, (3, Hq, D))).to(torch.bfloat16)
    n = bench.heavy_keys(pool, q, lay, 16, 40.0)
    # history positions 0, 16, ... below n - 1 of every sequence
    pos = [list(range(0, int(lay.seq_lens[s]) - 1, 16)) for s in range(3)]
    assert n == sum(len(p) for p in pos)
    u = q.float().view(3, Hkv, Hq // Hkv, D).sum(2)
    u = u / u.norm(dim=-1, keepdim=True)
    written = torch.zeros(pool.shape[:2], dtype=torch.bool)
    for s in range(3):
        for t in pos[s]:
            b, o = int(lay.block_tables[s, t // 16]), t % 16
            assert torch.equal(pool[b, o], (40.0 * u[s]).to(torch.bfloat16))
            written[b, o] = True
    assert (pool[~written] == 0).all()
