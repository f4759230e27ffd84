"""GPU parity of the mixture-of-experts GEMM fused with the combine
all-to-all (gsa_moe_gemm_all_to_all) through the C ABI, against the CPU
oracle's moe_combine.

Per call: every row the combine fills (in every rank's buffer) is within
|err| <= 1e-5 * sum_k |x_k w_k| + 1e-6 of the fp64 value; every other row of
every buffer is bit-identical to what it held before; flag (rank, e, t) is
the call's epoch in every pad and no other flag changed; repeated calls are
bit-identical.
"""
import sys

import numpy as np
import pytest
import torch

import gemv_shot_all_amd as gsa
import gsa_inputs as gi
import oracle
from tests.gpu_util import all_but, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


class MoeRun:
    def __init__(self, d, published_mask=None):
        self.d = d
        self.W, self.ne, self.H, self.F = d["W"], d["ne"], d["H"], d["F"]
        self.rank = d["rank"]
        self.rows_in, self.rows_out = d["rows_in"], d["rows_out"]
        self.X = to_dev(d["X"])
        self.Wd = to_dev(d["Wd"])
        self.splits = torch.from_numpy(
            np.concatenate([d["length"].ravel(), d["in_off"].ravel()]).astype(np.int32)).cuda()
        self.dst = torch.from_numpy(d["dst_off"].astype(np.int32).ravel()).cuda()
        self.buf = gsa.A2ABuffer(self.W, self.ne, self.H, self.rows_out)
        self.buf.bufs_view().copy_(torch.from_numpy(d["bufs"]).cuda())
        self.mask = all_but(self.W, self.rank) if published_mask is None else published_mask
        self.buf.reset(self.mask)
        torch.cuda.synchronize()

    def call(self):
        gsa.gsa_moe_gemm_all_to_all(self.X, self.Wd, self.splits, self.dst, self.buf.bufs,
                                    self.buf.pads, self.W, self.rank, self.ne, self.H, self.F,
                                    self.rows_in, self.rows_out)

    def results(self):
        torch.cuda.synchronize()
        return (self.buf.bufs_view().cpu().numpy(), self.buf.flags(),
                self.buf.status(self.rank))

    def close(self):
        self.buf.close()


def expected_flags(W, ne, tiles, rank, mask, epoch, experts=None):
    """W pads x W sources x ne x tiles after calls that raised `epoch` for
    this rank's experts (all, or those listed)."""
    f = np.zeros((W, W, ne, tiles), np.uint32)
    for p in range(W):
        if (mask >> p) & 1:
            f[:, p] = gsa.GSA_FLAG_PUBLISHED
    for e in (range(ne) if experts is None else experts):
        f[:, rank, e, :] = epoch
    return f


def check_moe(d, bufs_out, what, experts=None):
    """Rows of `experts` (default: all) within the bound of the oracle, every
    other row unchanged."""
    o = oracle.load()
    y64, abs64, written = o.moe_combine(d["X"], d["Wd"], d["length"], d["in_off"], d["dst_off"],
                                        d["W"], d["rows_out"])
    if experts is not None:  # only these experts' rows are expected written
        keep = np.zeros_like(written)
        for s in range(d["W"]):
            for e in experts:
                o_, n = int(d["dst_off"][s, e]), int(d["length"][e, s])
                keep[s, o_:o_ + n] = 1
        written = written & keep
    m = written.astype(bool)
    bnd = oracle.bound(abs64[m])
    err = np.abs(bufs_out[m].astype(np.float64) - y64[m])
    assert np.all(err <= bnd), f"{what}: max err/bound {np.max(err / bnd):.3g}"
    assert np.array_equal(bufs_out[~m].view(np.uint32), d["bufs"][~m].view(np.uint32)), (
        f"{what}: a row outside the combine's segments changed")
    return float(np.max(err / bnd)) if m.any() else 0.0


def run_moe_and_check(d, what):
    r = MoeRun(d)
    try:
        r.call()
        bufs, flags, status = r.results()
        tiles = r.buf.tiles
    finally:
        r.close()
    assert status == (gsa.GSA_OK, -1, -1), f"{what}: status {status}"
    check_moe(d, bufs, what)
    assert np.array_equal(flags, expected_flags(d["W"], d["ne"], tiles, d["rank"],
                                                all_but(d["W"], d["rank"]), 1)), f"{what}: flags"


@pytest.mark.parametrize("cfg", ["m0", "m1", "m2", "m3"])
def test_config_moe(cfg):
    _say(f"[moe] config {cfg}")
    run_moe_and_check(gi.make_moe_inputs(cfg, seed=0, rank=0), cfg)


def test_rank_sweep_moe():
    W = gi.MOE_CONFIGS["m1"]["W"]
    for rank in range(W):
        _say(f"[moe] m1 rank {rank}")
        run_moe_and_check(gi.make_moe_inputs("m1", seed=1, rank=rank), f"m1 rank {rank}")


def _counts(W, ne, rng, per_expert):
    """counts[s][g] with the given per-expert totals spread over source
    ranks at random."""
    E = W * ne
    counts = np.zeros((W, E), np.int64)
    for g in range(E):
        for _ in range(int(per_expert[g])):
            counts[int(rng.integers(0, W)), g] += 1
    return counts


EDGE = [
    # (W, ne, H, F, rank, tokens per expert (cycled), gap)
    (4, 3, 200, 64, 1, [16, 0, 5], 0),      # a full expert, an empty one, ragged H
    (2, 2, 16, 8, 0, [1, 16], 2),           # F = 8 (one chunk), gaps between segments
    (8, 2, 64, 4088, 7, [3, 16], 1),        # the widest F (x fills 128 KB of LDS)
    (1, 4, 48, 256, 0, [16, 1, 0, 7], 0),   # one rank
    (8, 1, 1000, 136, 3, [9], 0),           # ragged C, one expert per rank
    (3, 5, 33, 32, 2, [0], 0),              # no tokens at all
    (2, 2, 48, 2048, 1, [16, 2], 0),        # wide experts: two tiles per workgroup, 3 tiles
    (4, 2, 80, 1024, 3, [5], 1),            # four tiles per workgroup, 5 tiles
    (2, 2, 64, 256, 0, [17, 32], 0),        # one token past a 16-token tile; two whole tiles
    (4, 1, 80, 768, 2, [48], 1),            # three token tiles, gaps between segments
    (2, 2, 48, 2048, 1, [33, 0], 0),        # wide experts, three token tiles (the last of 1)
    (2, 1, 40, 64, 1, [256], 0),            # the most tokens an expert takes
    (2, 1, 48, 512, 0, [33], 0),            # two token tiles per weight pass, then a tile of 1
    (2, 1, 32, 960, 1, [40], 0),            # C = 120: one token tile per pass (LDS bound)
]


@pytest.mark.parametrize("W,ne,H,F,rank,per,gap", EDGE)
def test_edge_moe(W, ne, H, F, rank, per, gap):
    _say(f"[moe] edge W={W} ne={ne} H={H} F={F} rank={rank} per={per} gap={gap}")
    rng = np.random.default_rng(W * 1000 + ne * 100 + H + F)
    E = W * ne
    counts = _counts(W, ne, rng, [per[g % len(per)] for g in range(E)])
    d = gi.make_moe_from_counts(counts, ne, H, F, sigma=0.05, seed=9, cfg_id=H + F, rank=rank,
                                gap=gap)
    run_moe_and_check(d, f"W={W} ne={ne} H={H} F={F}")


def test_repeats_bit_identical():
    _say("[moe] repeats")
    d = gi.make_moe_inputs("m1", seed=3, rank=2)
    r = MoeRun(d)
    try:
        outs = []
        for i in range(3):
            r.call()
            bufs, flags, status = r.results()
            assert status == (gsa.GSA_OK, -1, -1)
            check_moe(d, bufs, f"call {i}")
            assert np.array_equal(flags, expected_flags(r.W, r.ne, r.buf.tiles, r.rank, r.mask,
                                                        i + 1))
            outs.append(bufs.copy())
    finally:
        r.close()
    for i in range(1, 3):
        assert np.array_equal(outs[i].view(np.uint32), outs[0].view(np.uint32))


def test_bad_split_table_is_reported_and_isolated():
    """Expert 1's table holds more tokens than it takes, expert 2's segment
    starts past X: both are reported (smallest expert first), write nothing
    and raise no flag; the other experts are unaffected."""
    _say("[moe] bad split tables")
    d = gi.make_moe_inputs("m0", seed=4, rank=1)
    ne, W = d["ne"], d["W"]
    d2 = dict(d)
    d2["length"] = d["length"].copy()
    d2["in_off"] = d["in_off"].copy()
    d2["length"][1, 0] = gsa.GSA_MOE_MAX_TOKENS + 1
    d2["in_off"][2, W - 1] = d["rows_in"] + 5
    r = MoeRun(d2)
    try:
        r.call()
        bufs, flags, status = r.results()
        tiles = r.buf.tiles
    finally:
        r.close()
    assert status == (gsa.GSA_ESPLIT, 1, -1), status
    good = [e for e in range(ne) if e not in (1, 2)]
    check_moe(d, bufs, "bad tables", experts=good)
    assert np.array_equal(flags, expected_flags(W, ne, tiles, d["rank"], all_but(W, d["rank"]), 1,
                                                experts=good))


def test_timeout_reports_missing_peer_and_still_delivers():
    """Rank 3's flags for expert 2 withheld in the own pad: those workgroups'
    waits expire (status names expert 2's first tile and rank 3), yet every
    row has been delivered and every flag of this rank raised."""
    _say("[moe] timeout")
    d = gi.make_moe_inputs("m0", seed=5, rank=0)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        r = MoeRun(d)
        try:
            pads = r.buf.pads_view()
            row = gsa.GSA_PAD_HEADER_WORDS + (3 * r.ne + 2) * r.buf.row_stride
            pads[r.rank, row:row + r.buf.row_stride] = 0
            torch.cuda.synchronize()
            r.call()
            bufs, flags, status = r.results()
            tiles = r.buf.tiles
        finally:
            r.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)
    assert status == (gsa.GSA_ETIMEOUT, 2 * tiles, 3), status
    check_moe(d, bufs, "timeout")
    want = expected_flags(d["W"], d["ne"], tiles, 0, all_but(d["W"], 0), 1)
    want[0, 3, 2, :] = 0
    assert np.array_equal(flags, want)


def test_own_row_marked_published_is_rejected():
    _say("[moe] own row published")
    d = gi.make_moe_inputs("m0", seed=6, rank=2)
    full = (1 << d["W"]) - 1
    r = MoeRun(d, published_mask=full)
    try:
        r.call()
        bufs, flags, status = r.results()
        tiles = r.buf.tiles
    finally:
        r.close()
    assert status == (gsa.GSA_ESTATE, 0, -1), status
    assert np.array_equal(bufs.view(np.uint32), d["bufs"].view(np.uint32)), "nothing written"
    assert np.all(flags == gsa.GSA_FLAG_PUBLISHED)
    assert tiles > 0


def test_graph_replays_match_eager():
    _say("[moe] graph replays")
    d = gi.make_moe_inputs("m1", seed=7, rank=5)
    r = MoeRun(d)
    try:
        r.call()
        b0, _, status = r.results()
        assert status == (gsa.GSA_OK, -1, -1)
        check_moe(d, b0, "eager")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(3):
                    r.call()
        for rep in range(3):
            g.replay()
            torch.cuda.synchronize()
            bufs, flags, status = r.results()
            assert status == (gsa.GSA_OK, -1, -1)
            assert np.array_equal(bufs.view(np.uint32), b0.view(np.uint32)), f"replay {rep}"
            assert np.array_equal(flags, expected_flags(r.W, r.ne, r.buf.tiles, r.rank, r.mask,
                                                        1 + 3 * (rep + 1)))
    finally:
        r.close()
