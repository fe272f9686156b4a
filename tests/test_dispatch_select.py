"""loka_dispatch_select (host only, through the C ABI) against the oracle's
Dispatch rule ([LoKA] section III-C, "Library and Recipe Selection") on
random candidate tables, plus its argument checks.  Runs on the CPU."""

import math

import numpy as np
import pytest

import fp8_precision_gemm_amd as lk
from oracle import dispatch


def test_matches_oracle_on_random_tables():
    rng = np.random.default_rng(0)
    for _ in range(3000):
        n = int(rng.integers(0, 7))
        us = rng.choice([rng.uniform(1.0, 20.0), 8.0, 9.5], size=n)
        mere = rng.choice([rng.uniform(0.0, 0.4), 0.2, 0.05], size=n)
        if n and rng.random() < 0.1:
            us[rng.integers(n)] = rng.choice([math.nan, math.inf, 0.0, -1.0])
        if n and rng.random() < 0.1:
            mere[rng.integers(n)] = rng.choice([math.nan, math.inf])
        base = float(rng.choice([10.0, rng.uniform(5.0, 25.0)]))
        mx = float(rng.choice([0.2, 0.1, 0.3]))
        sp = float(rng.choice([1.05, 1.0, 1.5]))
        cands = list(zip(us.tolist(), mere.tolist()))
        assert lk.loka_dispatch_select(cands, base, mx, sp) == dispatch.select(cands, base, mx, sp), (cands, base)


def test_pages_example_thresholds():
    # typical thresholds of the pages: MERE < 0.2, speedup > 1.05x
    assert lk.loka_dispatch_select([(5.0, 0.25), (7.0, 0.1), (9.7, 0.0)], 10.0) == 1
    assert lk.loka_dispatch_select([(9.7, 0.0)], 10.0) == -1


@pytest.mark.parametrize("args", [
    ([(1.0, 0.0)], 0.0, 0.2, 1.05), ([(1.0, 0.0)], math.nan, 0.2, 1.05), ([(1.0, 0.0)], 10.0, 0.0, 1.05),
    ([(1.0, 0.0)], 10.0, 0.2, -1.0), ([(1.0, 0.0)], 10.0, math.inf, 1.05),
])
def test_rejects_bad_arguments(args):
    with pytest.raises(lk.LokaError):
        lk.loka_dispatch_select(*args)
