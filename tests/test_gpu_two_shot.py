"""GPU parity of the two-shot variant (gsa_gemv_allreduce_two_shot) through
the C ABI, against the CPU oracle.

Per call: the published slot is within the fp64 bound; out is bit-identical
to the oracle's two-shot result from the slots as read back and the seeded
gathered rows (own chunk: the rank-order fp32 fold, within the fp64 bound
too; every other row: the owner's gathered row, copied exactly); the own
chunk's rows of `gathered` hold exactly the published values and no other
row of it changes; peer slots are untouched; slot flags and reduced-chunk
flags advance as the protocol says.
"""
import sys

import numpy as np
import pytest
import torch

import gemv_shot_all_amd as gsa
import gsa_inputs as gi
import oracle
from tests.gpu_util import Run, all_but, check_against_oracle, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def own_rows(N, W, rank):
    c = oracle.load().two_shot_chunk_rows(N, W)
    return slice(min(N, rank * c), min(N, (rank + 1) * c))


def own_tiles(N, W, rank):
    rows = own_rows(N, W, rank)
    T = oracle.flag_tiles(N)
    return [t for t in range(T) if rows.start <= oracle.FLAG_TILE_ROWS * t < rows.stop]


class TwoShotRun:
    def __init__(self, d, rank=None, seed=0, published_mask=None):
        self.d = d
        self.rank = d["rank"] if rank is None else rank
        self.slots_in = d["slots"].copy()
        self.r = Run(d["A"], d["x"], self.slots_in, self.rank, published_mask)
        N, B, W = self.r.N, self.r.B, self.r.W
        g = gi.make_gathered(N, B, seed=seed, cfg_id=1000 + N + B)
        g[own_rows(N, W, self.rank)] = gi.sentinel((B,))
        self.gathered_in = g
        self.r.buf.gathered_view().copy_(to_dev(g))
        torch.cuda.synchronize()

    def call(self):
        r = self.r
        gsa.gsa_gemv_allreduce_two_shot(r.A, r.x, r.buf.slots, r.buf.pad, r.buf.gathered, r.out,
                                        r.W, self.rank, r.N, r.K, r.B)

    def results(self):
        out, slots, flags, status = self.r.results()
        return (out, slots, self.r.buf.gathered_view().cpu().numpy(), flags,
                self.r.buf.flags2(), status)

    def close(self):
        self.r.close()


def check_two_shot(ts, out, slots_out, gathered_out, what):
    d, rank = ts.d, ts.rank
    W, N, B = slots_out.shape
    o = oracle.load()
    expect, mine = o.two_shot(slots_out, ts.gathered_in, rank)
    assert np.array_equal(out.view(np.uint32), expect.view(np.uint32)), (
        f"{what}: out differs from the two-shot result (own chunk fold, other rows copied)")
    rows = own_rows(N, W, rank)
    # the own chunk within the fp64 bound, and the slot / peer-slot checks
    y64, abs64, out64 = o.gemv_allreduce(d["A"], d["x"], ts.slots_in, rank)
    bnd = oracle.bound(abs64)
    assert np.all(np.abs(out[rows].astype(np.float64) - out64[rows]) <= bnd[rows]), (
        f"{what}: own chunk off the fp64 bound")
    assert np.all(np.abs(slots_out[rank].astype(np.float64) - y64) <= bnd), (
        f"{what}: published slot off the fp64 bound")
    for p in range(W):
        if p != rank:
            assert np.array_equal(slots_out[p].view(np.uint32), ts.slots_in[p].view(np.uint32))
    # gathered: own rows = the published values, the rest untouched
    want = ts.gathered_in.copy()
    want[rows] = mine[rows]
    assert np.array_equal(gathered_out.view(np.uint32), want.view(np.uint32)), (
        f"{what}: gathered rows")


def expected_flags2(W, N, rank, mask, epoch_of_last_two_shot):
    f2 = oracle.pad_after_reset(W, N, mask)
    for t in own_tiles(N, W, rank):
        f2[rank, t] = epoch_of_last_two_shot
    return f2


def run_two_shot_and_check(d, what, rank=None, seed=0):
    ts = TwoShotRun(d, rank=rank, seed=seed)
    try:
        ts.call()
        out, sl, g, flags, flags2, status = ts.results()
    finally:
        ts.close()
    assert status == (gsa.GSA_OK, -1, -1), f"{what}: status {status}"
    check_two_shot(ts, out, sl, g, what)
    W, N = sl.shape[0], sl.shape[1]
    mask = all_but(W, ts.rank)
    assert np.array_equal(flags, oracle.pad_after_calls(oracle.pad_after_reset(W, N, mask),
                                                        ts.rank, 1)), f"{what}: slot flags"
    assert np.array_equal(flags2, expected_flags2(W, N, ts.rank, mask, 1)), (
        f"{what}: reduced-chunk flags")


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3b1", "c3b4", "c3b8", "c4", "c5"])
def test_config_two_shot(cfg):
    _say(f"[two-shot] config {cfg}")
    d = gi.make_inputs(cfg, seed=0, rank=0)
    run_two_shot_and_check(d, cfg)


@pytest.mark.parametrize("cfg", ["c2", "c5"])
def test_rank_sweep_two_shot(cfg):
    W = gi.CONFIGS[cfg]["W"]
    for rank in range(W):
        _say(f"[two-shot] config {cfg} rank {rank}")
        d = gi.make_inputs(cfg, seed=1, rank=rank)
        run_two_shot_and_check(d, f"{cfg} rank {rank}", seed=rank)


EDGE = [
    # (W, N, Ks, B, rank)
    (2, 1000, 512, 1, 1),        # ragged N, the last chunk short
    (8, 17, 512, 3, 0),          # 2 tiles: ranks 0 and 1 own one each
    (8, 17, 512, 3, 1),          # ... the owner of the one-row tile
    (8, 17, 512, 3, 5),          # ... a rank that owns nothing
    (1, 1, 8, 1, 0),             # one rank, one row
    (3, 100, 64, 2, 2),          # chunk 48 rows: rank 2 owns 4 rows
    (4, 50, 2048, 9, 3),         # MFMA, ragged: rank 3 owns nothing
    (4, 4000, 256, 16, 1),       # MFMA, 250 tiles
    (8, 8192 + 16 * 65, 64, 2, 7),  # 577 tiles, short rows, the last chunk short
    (2, 16 * 6000 + 5, 64, 3, 1),   # 6001 tiles, ragged
    (2, 32, 8192, 8, 1),         # x at the LDS bound (128 KB)
    (8, 40, 65536, 12, 3),       # MFMA, 1.5 MB of x (read from memory), ragged N
    (8, 300, 1024, 7, 6),        # long tier, B = 7
]


@pytest.mark.parametrize("W,N,Ks,B,rank", EDGE)
def test_edge_two_shot(W, N, Ks, B, rank):
    _say(f"[two-shot] edge W={W} N={N} Ks={Ks} B={B} rank={rank}")
    d = gi.make_shard_inputs(W, N, Ks, B, sigma=0.02, seed=7, cfg_id=4000 + N + B, rank=rank)
    run_two_shot_and_check(d, f"W={W} N={N} Ks={Ks} B={B} rank={rank}", seed=3)


@pytest.mark.parametrize("cfg", ["c3b4", "c2"])  # 16-row and 4-row workgroups
def test_repeats_and_mixed_with_plain_calls(cfg):
    """two-shot, plain, two-shot, plain, two-shot on one buffer: every
    two-shot call gives the same bits; slot flags count every call; the
    reduced-chunk flags of the own chunk carry the last two-shot call's
    epoch."""
    _say(f"[two-shot] repeats mixed with plain calls, {cfg}")
    d = gi.make_inputs(cfg, seed=2, rank=3)
    ts = TwoShotRun(d, seed=2)
    W, N = ts.r.W, ts.r.N
    try:
        outs = []
        for i in range(3):
            ts.call()
            out, sl, g, flags, flags2, status = ts.results()
            assert status == (gsa.GSA_OK, -1, -1)
            check_two_shot(ts, out, sl, g, f"call {i}")
            outs.append(out.copy())
            epoch = 2 * i + 1
            mask = all_but(W, ts.rank)
            assert np.array_equal(flags, oracle.pad_after_calls(
                oracle.pad_after_reset(W, N, mask), ts.rank, epoch))
            assert np.array_equal(flags2, expected_flags2(W, N, ts.rank, mask, epoch))
            if i < 2:
                ts.r.call()  # a plain one-shot call in between
                o_plain, sl2, _, st = ts.r.results()
                assert st == (gsa.GSA_OK, -1, -1)
                check_against_oracle(d["A"], d["x"], ts.slots_in, ts.rank, o_plain, sl2,
                                     f"plain call {i}")
    finally:
        ts.close()
    for i in range(1, 3):
        assert np.array_equal(outs[i].view(np.uint32), outs[0].view(np.uint32))


def test_timeout_withheld_slot_flag():
    """Peer 2's slot flags withheld: this rank's own chunk cannot be reduced
    (status names its first tile and peer 2; those out rows, the gathered
    rows and the reduced-chunk flags stay untouched); every other chunk is
    copied from its owner as usual."""
    _say("[two-shot] timeout, slot flags of a peer withheld")
    W, rank, N, B = 4, 1, 200, 2
    d = gi.make_shard_inputs(W, N, 256, B, seed=13, rank=rank)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        ts = TwoShotRun(d, seed=13)
        try:
            pad = ts.r.buf.pad_view()
            pad[gsa.GSA_PAD_HEADER_WORDS + 2 * ts.r.buf.row_stride:
                gsa.GSA_PAD_HEADER_WORDS + 3 * ts.r.buf.row_stride] = 0
            torch.cuda.synchronize()
            ts.call()
            out, sl, g, flags, flags2, status = ts.results()
        finally:
            ts.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)
    tiles = own_tiles(N, W, rank)
    assert status == (gsa.GSA_ETIMEOUT, tiles[0], 2), status
    rows = own_rows(N, W, rank)
    assert np.isnan(out[rows]).all(), "timed-out tiles must not write out"
    rest = np.ones(N, bool)
    rest[rows] = False
    assert np.array_equal(out[rest].view(np.uint32), ts.gathered_in[rest].view(np.uint32))
    assert np.array_equal(g.view(np.uint32), ts.gathered_in.view(np.uint32))
    assert np.all(flags2[rank] == 0)
    y64, abs64, _ = oracle.load().gemv_allreduce(d["A"], d["x"], d["slots"], rank)
    assert np.all(np.abs(sl[rank] - y64) <= oracle.bound(abs64)), "own slot must be published"


def test_timeout_withheld_reduced_chunk_flag():
    """Owner 3's reduced-chunk flags withheld: only its chunk times out
    (status names its first tile and peer 3); the own chunk is reduced and
    published, the other chunks copied."""
    _say("[two-shot] timeout, reduced-chunk flags of an owner withheld")
    W, rank, N, B = 4, 0, 200, 2
    d = gi.make_shard_inputs(W, N, 256, B, seed=14, rank=rank)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        ts = TwoShotRun(d, seed=14)
        try:
            rs = ts.r.buf.row_stride
            pad = ts.r.buf.pad_view()
            pad[gsa.GSA_PAD_HEADER_WORDS + (W + 3) * rs:gsa.GSA_PAD_HEADER_WORDS + (W + 4) * rs] = 0
            torch.cuda.synchronize()
            ts.call()
            out, sl, g, flags, flags2, status = ts.results()
        finally:
            ts.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)
    assert status == (gsa.GSA_ETIMEOUT, own_tiles(N, W, 3)[0], 3), status
    bad = own_rows(N, W, 3)
    assert np.isnan(out[bad]).all()
    o = oracle.load()
    expect, mine = o.two_shot(sl, ts.gathered_in, rank)
    good = np.ones(N, bool)
    good[bad] = False
    assert np.array_equal(out[good].view(np.uint32), expect[good].view(np.uint32))
    mr = own_rows(N, W, rank)
    assert np.array_equal(g[mr].view(np.uint32), mine[mr].view(np.uint32))
    assert all(flags2[rank, t] == 1 for t in own_tiles(N, W, rank))


def test_graph_replays_match_eager():
    """Calls captured in a HIP graph: every replay gives the eager result,
    bit for bit, and the flags keep counting."""
    _say("[two-shot] graph replays")
    d = gi.make_inputs("c2", seed=5, rank=6)
    ts = TwoShotRun(d, seed=5)
    try:
        ts.call()
        out0, sl0, g0, _, _, status = ts.results()
        assert status == (gsa.GSA_OK, -1, -1)
        check_two_shot(ts, out0, sl0, g0, "eager")
        gr = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(gr, stream=s):
                for _ in range(3):
                    ts.call()
        for rep in range(3):
            ts.r.out.fill_(float("nan"))
            gr.replay()
            torch.cuda.synchronize()
            out, sl, g, flags, flags2, status = ts.results()
            assert status == (gsa.GSA_OK, -1, -1)
            assert np.array_equal(out.view(np.uint32), out0.view(np.uint32)), f"replay {rep}"
            assert np.array_equal(g.view(np.uint32), g0.view(np.uint32)), f"replay {rep}"
            assert np.all(flags[ts.rank] == 1 + 3 * (rep + 1))
    finally:
        ts.close()
