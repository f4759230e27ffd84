"""A seeded sweep of random shapes through every GEMV entry point (needs an
MI355X), each checked to the same bar as the named workloads and edges:
the plain call against the oracle, the element-type call in a random slot /
out combination, the fused bias + RMSNorm epilogue and the two-shot variant.

The shapes are drawn once from a fixed seed (W in 1..8, rank < W, N in
1..6000, B in 1..16, rows of C = Ks / 8 chunks, with the chunk counts that
select a kernel of their own drawn more often), so the sweep is the same
on every run; each case prints its shape before it runs."""
import sys

import numpy as np
import pytest
import torch

import gemv_shot_all_amd as gsa
import gsa_inputs as gi
from tests.gpu_util import run_and_check
from tests.test_gpu_dtype import DRun, check_dtype_call
from tests.test_gpu_epilogue import run_epi_and_check
from tests.test_gpu_two_shot import run_two_shot_and_check

pytestmark = pytest.mark.gpu

F32, BF16 = gsa.GSA_DTYPE_F32, gsa.GSA_DTYPE_BF16
# Chunk counts at the tier bounds and of the unrolled instances: 64 (short
# rows), 224 (the middle tier's unrolled rows), 225, 256 (the LDS-staged
# MFMA kernel), 448 (the long-row kernel's unrolled rows).
SPECIAL_C = [1, 8, 63, 64, 65, 224, 225, 256, 448, 449]
MAX_WORK = 48 << 20  # N * Ks * B, so that the oracle finishes in about a second


def _cases(n, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        W = int(rng.integers(1, 9))
        rank = int(rng.integers(0, W))
        B = int(rng.integers(1, 17))
        C = int(rng.choice(SPECIAL_C)) if rng.random() < 0.5 else int(rng.integers(1, 1025))
        N = int(rng.integers(1, 6001))
        Ks = 8 * C
        if N * Ks * B > MAX_WORK:
            N = max(1, MAX_WORK // (Ks * B))
        out.append((W, N, Ks, B, rank))
    return out


# Drawn, then the chunk counts the draw missed: the LDS-staged MFMA rows
# (256 chunks, B > 8), one-chunk rows and the long rows just past the
# unrolled instance.
CASES = _cases(48) + [(4, 1000, 2048, 12, 1), (2, 77, 2048, 16, 0), (8, 300, 8, 3, 5),
                      (3, 500, 3592, 4, 2)]


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _inputs(case, i):
    W, N, Ks, B, rank = case
    return gi.make_shard_inputs(W, N, Ks, B, sigma=0.02, seed=40 + i, cfg_id=9000 + i, rank=rank)


def _id(case):
    W, N, Ks, B, rank = case
    return f"W{W}-N{N}-Ks{Ks}-B{B}-r{rank}"


@pytest.mark.parametrize("i,case", list(enumerate(CASES)), ids=[_id(c) for c in CASES])
def test_sweep_plain_and_dtype(i, case):
    _say(f"[sweep] plain + dtype {_id(case)}")
    d = _inputs(case, i)
    run_and_check(d, what=_id(case))
    dts = [(BF16, BF16), (BF16, F32), (F32, BF16)][i % 3]
    r = DRun(d, case[4], *dts)
    try:
        r.call()
        res = r.results()
    finally:
        r.close()
    check_dtype_call(r, *res, what=f"{_id(case)} dtypes {dts}")


@pytest.mark.parametrize("i,case", list(enumerate(CASES)), ids=[_id(c) for c in CASES])
def test_sweep_epilogue_and_two_shot(i, case):
    _say(f"[sweep] epilogue + two-shot {_id(case)}")
    d = _inputs(case, i)
    run_epi_and_check(d, _id(case), bias=(i % 2 == 0), weight=(i % 3 != 0),
                      eps=[1e-5, 1e-6, 1e-3][i % 3],
                      y_dtype=torch.bfloat16 if i % 2 else torch.float32)
    run_two_shot_and_check(d, _id(case), seed=i)
