"""Parity of the HIP path with the CPU oracle (needs an MI355X).

Every named workload at full size, plus ragged and degenerate shapes that
exercise each kernel tier, the masked chunk paths, the MFMA path and the
multi-pass loops."""
import sys

import numpy as np
import pytest

import gsa_inputs as gi
from tests.gpu_util import run_and_check

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.mark.parametrize("cfg", list(gi.CONFIGS))
def test_config_parity(cfg):
    _say(f"[parity] config {cfg}")
    d = gi.make_inputs(cfg, seed=0, rank=0)
    ratio = run_and_check(d, what=cfg)
    _say(f"[parity] {cfg}: max err/bound out {ratio[0]:.3g} slot {ratio[1]:.3g}")


EDGE = [
    # (W, N, Ks, B, rank)
    (2, 1000, 512, 1, 1),     # ragged N, short rows
    (8, 17, 512, 3, 7),       # one full tile + 1 row
    (1, 1, 8, 1, 0),          # smallest: one row, one chunk, W = 1
    (3, 40, 24, 2, 1),        # C = 3 (masked short tier)
    (4, 64, 1800, 4, 2),      # C = 225: long tier, masked
    (8, 100, 1792, 8, 3),     # down_proj rows, B = 8
    (2, 48, 16384, 1, 0),     # multi-pass long rows
    (2, 32, 8192, 8, 1),      # x at the LDS bound (128 KB)
    (2, 33, 5000, 5, 0),      # masked multi-pass, B = 5
    (4, 50, 2048, 9, 3),      # MFMA path, A staged through LDS, B = 9, ragged N
    (8, 4099, 2048, 16, 7),   # the same, W = 8, last rank, 129 workgroups, the last of 3 rows
    (1, 31, 2048, 13, 0),     # the same, W = 1, one partial workgroup
    (2, 33, 2048, 16, 1),     # the same, a second workgroup of one row
    (8, 1, 2048, 10, 0),      # the same, a single row
    (4, 64, 200, 16, 1),      # MFMA, C = 25 (masked)
    (2, 16, 8, 16, 0),        # MFMA, single chunk
    (8, 128, 4000, 12, 5),    # MFMA multi-pass, masked
    (1, 70, 256, 16, 0),      # MFMA, W = 1
    (2, 32, 8192, 16, 1),     # MFMA, x 256 KB (read from memory, not staged)
    (8, 40, 65536, 12, 3),    # MFMA, 1.5 MB of x, ragged N
    (4, 24, 72, 10, 0),       # MFMA, C = 9: fewer k-steps than waves
    (8, 4096, 512, 6, 4),     # short tier, B = 6
    (4, 123, 512, 8, 2),      # 4-row tiles, B = 8, the last tile 3 rows
    (2, 6, 64, 7, 1),         # 4-row tiles, C = 8, the second tile 2 rows
    (8, 300, 1024, 7, 6),     # long tier, B = 7
]


@pytest.mark.parametrize("W,N,Ks,B,rank", EDGE)
def test_edge_shape_parity(W, N, Ks, B, rank):
    _say(f"[parity] edge W={W} N={N} Ks={Ks} B={B} rank={rank}")
    d = gi.make_shard_inputs(W, N, Ks, B, sigma=0.02, seed=1, cfg_id=1000 + N + Ks + B,
                             rank=rank)
    run_and_check(d, what=f"W={W} N={N} Ks={Ks} B={B}")


@pytest.mark.parametrize("B", list(range(1, 17)))
def test_every_batch_size(B):
    _say(f"[parity] B={B}")
    d = gi.make_shard_inputs(4, 96, 1792, B, sigma=0.02, seed=2, cfg_id=2000 + B, rank=2)
    run_and_check(d, what=f"B={B}")
