"""The division step of the E4M3 V store (scales in [2^-64, 2^64]): from the
host's correctly rounded reciprocal r = RN(1/d), q0 = RN(x r) and one fused
residual correction give the IEEE quotient x / d bit for bit wherever the
quotient's E4M3 code depends on its rounding (|x / d| in [2^-12, 2^10]), for
divisors across and at the ends of that range, an all-ones significand
among them (for the kernel's d, an exhaustive run over all 2^32 x found no
E4M3 code differing).  CPU only: the step is compiled with gcc from
tests/div_by_scale_check.c (fmaf is the fused, correctly rounded
operation the kernel's v_fma_f32 computes)."""
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("div") / "div_by_scale_check")
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-std=c11",
                    os.path.join(HERE, "div_by_scale_check.c"), "-o", exe, "-lm"], check=True)
    return exe


def test_division_step_matches_ieee_division(checker):
    f32 = lambda v: float(np.float32(v))
    ds = [1.0, 3.0, f32(0.0364877), f32(31.999998092651367), 0.01, 1 / 3, 0.37, 65535.0,
          f32(0.99999994), 2.0 ** -64, f32(2.0 ** -64 * 1.9999998), 2.0 ** 64,
          f32(2.0 ** 63 * 1.9999998), f32(2.0 ** -40 * 1.7), f32(2.0 ** 40 * 1.1)]
    rng = np.random.default_rng(5)
    ds += [f32(v) for v in np.exp(rng.uniform(np.log(2.0 ** -64), np.log(2.0 ** 64), 10))]
    inp = "".join(f"{d!r} 200000 {i + 1}\n" for i, d in enumerate(ds))
    out = subprocess.run([checker], input=inp.encode(), stdout=subprocess.PIPE,
                         check=True).stdout.decode().split("\n")
    rows = [line.split() for line in out if line.strip()]
    assert len(rows) == len(ds)
    for d, n, bad in rows:
        assert int(n) > 200000 and int(bad) == 0, (d, n, bad)
