"""The launch contract of the C ABI, observed with rocprofv3 (HIP API,
kernel-dispatch, memory-copy and marker traces of
tests/launch_contract_child.py):

* a call with no work (zero tokens or sequences) launches nothing: no HIP
  API call inside its range launches, copies, sets, allocates, frees or
  synchronises, and no kernel dispatch comes from it (page 1, kv_cache.rs,
  fill_slots_from_block_table returns before launching when the count is 0);
* a call with work, on inputs already on the device, launches only the
  library's kernels and issues no memory copy, memset, allocation, free or
  synchronisation (page 3, mla_cuda.rs: the device-resident KV path moves
  only the output back to the host; here every output stays on the device).
"""
import csv
import os
import shutil
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
FORBIDDEN = ("Memcpy", "Memset", "Malloc", "Free", "Synchronize", "HostRegister", "MemAlloc",
             "MallocAsync", "MemPool")


def _rows(path):
    if not os.path.exists(path):
        return []
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


@pytest.fixture(scope="module")
def trace(tmp_path_factory):
    prof = shutil.which("rocprofv3")
    if prof is None:
        pytest.skip("rocprofv3 not found")
    out = str(tmp_path_factory.mktemp("launch_contract"))
    env = dict(os.environ, TMPDIR="/tmp")
    cmd = [prof, "--hip-trace", "--kernel-trace", "--memory-copy-trace", "--marker-trace",
           "--output-format", "csv", "-d", out, "-o", "t", "--",
           sys.executable, os.path.join(HERE, "launch_contract_child.py")]
    print("running the launch-contract child under rocprofv3", flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT,
                       timeout=240)
    text = r.stdout.decode(errors="replace")
    assert r.returncode == 0 and "launch contract child" in text, text[-3000:]
    t = {k: _rows(os.path.join(out, f"t_{k}.csv"))
         for k in ("marker_api_trace", "hip_api_trace", "kernel_trace", "memory_copy_trace")}
    ranges = {row["Function"]: row for row in t["marker_api_trace"]}
    assert {"pkv_zero_work", "pkv_calls"} <= set(ranges), list(ranges)
    return t, ranges


def _in_range(t, rng):
    """HIP API calls of the range's thread inside the range, and the kernel
    dispatches and memory copies they caused (by correlation id)."""
    lo, hi, tid = int(rng["Start_Timestamp"]), int(rng["End_Timestamp"]), rng["Thread_Id"]
    api = [a for a in t["hip_api_trace"]
           if a["Domain"].startswith("HIP") and a["Thread_Id"] == tid
           and lo <= int(a["Start_Timestamp"]) and int(a["End_Timestamp"]) <= hi]
    corr = {a["Correlation_Id"] for a in api}
    kernels = [k for k in t["kernel_trace"] if k["Correlation_Id"] in corr]
    copies = [c for c in t["memory_copy_trace"] if c["Correlation_Id"] in corr]
    return api, kernels, copies


def test_zero_work_calls_launch_nothing(trace):
    t, ranges = trace
    api, kernels, copies = _in_range(t, ranges["pkv_zero_work"])
    names = sorted({a["Function"] for a in api})
    print(f"HIP API calls in the zero-work range: {names}")
    assert not kernels, [k["Kernel_Name"][:80] for k in kernels]
    assert not copies
    bad = [n for n in names if "Launch" in n or any(f in n for f in FORBIDDEN)]
    assert not bad, bad


def test_calls_launch_only_library_kernels_and_copy_nothing(trace):
    t, ranges = trace
    api, kernels, copies = _in_range(t, ranges["pkv_calls"])
    names = sorted({a["Function"] for a in api})
    print(f"HIP API calls in the calls range: {names}")
    print(f"{len(kernels)} kernels: {sorted({k['Kernel_Name'].split('(')[0][:60] for k in kernels})}")
    bad = [n for n in names if any(f in n for f in FORBIDDEN)]
    assert not bad, bad
    assert not copies, copies[:3]
    # eleven calls: slots, two K writes, two V writes, three decodes (one
    # with the sparse-V skip) and the no-allocation decode (split kernel and
    # merge each), prefill, MLA rows
    assert len(kernels) >= 11
    assert all("pkv::" in k["Kernel_Name"] for k in kernels), \
        [k["Kernel_Name"][:80] for k in kernels if "pkv::" not in k["Kernel_Name"]]
