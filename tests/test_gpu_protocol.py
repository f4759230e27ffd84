"""The fused call's protocol and closed forms on the GPU (needs an MI355X):
determinism, flag state, the W = 1 and shard-sum identities, closed-form
inputs with exact results, rank sweep, timeouts and a bad own flag row
(forced from the host with a short wait bound), graph replays."""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import gemv_shot_all_amd as gsa
import gsa_inputs as gi
import oracle
from tests.gpu_util import Run, all_but, check_against_oracle, run_and_check, to_dev

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint32)


REPEATS = 100


@pytest.mark.parametrize("cfg", ["c2", "c3b8", "c4", "c5"])
def test_repeats_bit_identical_and_flag_epochs(cfg):
    """REPEATS calls on one buffer: out and every slot byte-identical to the
    first call's, and the own flags count the calls."""
    _say(f"[protocol] repeats {cfg}")
    d = gi.make_inputs(cfg, seed=3)
    r = Run(d["A"], d["x"], d["slots"].copy(), 0)
    try:
        r.call()
        out0, sl0, _, _ = r.results()
        for i in range(1, REPEATS):
            r.out.fill_(float("nan"))
            r.call()
            out, sl, flags, status = r.results()
            assert np.array_equal(_bits(out), _bits(out0)), f"out differs at call {i}"
            assert np.array_equal(_bits(sl), _bits(sl0)), f"slots differ at call {i}"
        assert status == (gsa.GSA_OK, -1, -1)
        expect = oracle.pad_after_calls(oracle.pad_after_reset(d["W"], d["N"], all_but(d["W"], 0)),
                                        0, REPEATS)
        assert np.array_equal(flags, expect), "own flags must count the calls"
    finally:
        r.close()


def test_bit_identical_across_buffers_and_streams():
    _say("[protocol] across buffers/streams")
    d = gi.make_inputs("c3b4", seed=4)
    r1 = Run(d["A"], d["x"], d["slots"].copy(), 0)
    r2 = Run(d["A"], d["x"], d["slots"].copy(), 0)
    try:
        r1.call()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            r2.call()
        torch.cuda.synchronize()
        o1, s1, _, _ = r1.results()
        o2, s2, _, _ = r2.results()
        assert np.array_equal(_bits(o1), _bits(o2)) and np.array_equal(_bits(s1), _bits(s2))
    finally:
        r1.close()
        r2.close()


_CHILD = """
import sys
import numpy as np
import gsa_inputs as gi
from tests.gpu_util import Run
d = gi.make_inputs("c3b4", seed=4)
r = Run(d["A"], d["x"], d["slots"].copy(), 0)
r.call()
out, sl, flags, status = r.results()
r.close()
np.savez(sys.argv[1], out=out, slots=sl, flags=flags, status=np.array(status))
"""


def test_bit_identical_across_processes(tmp_path):
    """The same call in a second process (started after this one's calls):
    out, every slot and the flags byte-identical, status clean in both."""
    _say("[protocol] across processes")
    d = gi.make_inputs("c3b4", seed=4)
    r = Run(d["A"], d["x"], d["slots"].copy(), 0)
    try:
        r.call()
        out, sl, flags, status = r.results()
    finally:
        r.close()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = str(tmp_path / "child.npz")
    child = subprocess.run([sys.executable, "-c", _CHILD, path], cwd=root, timeout=300,
                           capture_output=True, text=True)
    assert child.returncode == 0, child.stderr[-2000:]
    got = np.load(path)
    assert status == (gsa.GSA_OK, -1, -1) and tuple(got["status"]) == status
    assert np.array_equal(_bits(got["out"]), _bits(out)), "out differs between processes"
    assert np.array_equal(_bits(got["slots"]), _bits(sl)), "slots differ between processes"
    assert np.array_equal(got["flags"], flags)


@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_rank_sweep(cfg):
    W = gi.CONFIGS[cfg]["W"]
    for rank in range(W):
        _say(f"[protocol] {cfg} rank {rank}")
        d = gi.make_inputs(cfg, seed=5, rank=rank)
        run_and_check(d, rank=rank, what=f"{cfg} rank {rank}")


@pytest.mark.parametrize("B", [1, 4, 8, 16])
def test_single_rank_equals_unsharded_gemv(B):
    _say(f"[protocol] W=1 B={B}")
    A, x = gi.make_full_inputs(160, 1024, B, sigma=0.02, seed=6)
    slots = np.full((1, 160, B), np.nan, np.float32)
    r = Run(A, x, slots, 0)
    try:
        r.call()
        out, sl, _, status = r.results()
    finally:
        r.close()
    assert status == (gsa.GSA_OK, -1, -1)
    assert np.array_equal(_bits(out), _bits(sl[0])), "W=1: out must equal the published slot"
    y64, abs64 = oracle.load().gemv(A, x)
    assert np.all(np.abs(out - y64) <= oracle.bound(abs64))


@pytest.mark.parametrize("W,B", [(2, 1), (8, 4), (4, 16)])
def test_sequential_shards_sum_to_full_gemv(W, B):
    """Run every rank's call on one GPU in turn: ranks 1..W-1 publish their
    partials (the others marked published), then rank 0's one-shot sum must
    equal the unsharded product within the bound over the full K."""
    _say(f"[protocol] shard sum W={W} B={B}")
    N, K = 96, 512 * W
    A, x = gi.make_full_inputs(N, K, B, sigma=0.02, seed=7)
    buf = gsa.SymmBuffer(W, N, B)
    out = torch.full((N, B), float("nan"), dtype=torch.float32, device="cuda")
    try:
        buf.slots_view().fill_(float("nan"))
        for r in list(range(1, W)) + [0]:
            Ar, xr = gi.shard(A, x, W, r)
            buf.reset(all_but(W, r))
            gsa.gsa_gemv_allreduce(to_dev(Ar), to_dev(xr), buf.slots, buf.pad, out, W, r, N, K, B)
        torch.cuda.synchronize()
        assert buf.status()[0] == gsa.GSA_OK
        got = out.cpu().numpy()
        slots = buf.slots_view().cpu().numpy()
    finally:
        buf.close()
    y64, abs64 = oracle.load().gemv(A, x)
    assert np.all(np.abs(got - y64) <= oracle.bound(abs64)), "shard sum != full GEMV"
    assert np.array_equal(_bits(got), _bits(oracle.load().fold_f32(slots)))


def _exact_case(A_vals, x_vals, W, rank, peers_int):
    N, Ks = A_vals.shape
    B = x_vals.shape[0]
    A = gi.bf16_bits(A_vals.astype(np.float32))
    x = gi.bf16_bits(x_vals.astype(np.float32))
    slots = np.zeros((W, N, B), np.float32)
    for r in range(W):
        slots[r] = peers_int[r]
    slots[rank] = np.nan
    r = Run(A, x, slots.copy(), rank)
    try:
        r.call()
        out, sl, _, status = r.results()
    finally:
        r.close()
    assert status == (gsa.GSA_OK, -1, -1)
    return out, sl


@pytest.mark.parametrize("B", [1, 3, 8, 16])
def test_closed_form_identity_and_integers(B):
    """Exact in any summation order: A = I gives y = x; small integers give
    exact integer sums (|partial sums| < 2^24)."""
    _say(f"[protocol] closed forms B={B}")
    rng = np.random.default_rng(8)
    Ks = 256
    xi = rng.integers(-4, 5, (B, Ks))
    W, rank = 4, 2
    peers = [rng.integers(-8, 9, (Ks, B)) for _ in range(W)]
    out, sl = _exact_case(np.eye(Ks), xi, W, rank, peers)
    assert np.array_equal(sl[rank], xi.T.astype(np.float32)), "identity: y != x"
    expect = xi.T + sum(peers[r] for r in range(W) if r != rank)
    assert np.array_equal(out, expect.astype(np.float32))
    N = 40
    Ai = rng.integers(-4, 5, (N, Ks))
    peers = [rng.integers(-8, 9, (N, B)) for _ in range(W)]
    out, sl = _exact_case(Ai, xi, W, rank, peers)
    assert np.array_equal(sl[rank], (Ai @ xi.T).astype(np.float32)), "integer GEMV inexact"
    expect = Ai @ xi.T + sum(peers[r] for r in range(W) if r != rank)
    assert np.array_equal(out, expect.astype(np.float32))


@pytest.mark.parametrize("B", [2, 16])
def test_closed_form_one_hot(B):
    """x_b = e_{j_b} picks column j_b of A exactly (catches operand and
    accumulator layout mistakes, MFMA path included)."""
    _say(f"[protocol] one-hot B={B}")
    rng = np.random.default_rng(9)
    N, Ks = 48, 512
    A = rng.normal(0, 1, (N, Ks))
    cols = rng.choice(Ks, B, replace=False)
    xv = np.zeros((B, Ks))
    xv[np.arange(B), cols] = 1.0
    out, sl = _exact_case(A, xv, 1, 0, [np.zeros((N, B))])
    Af = gi.bf16_bits_to_f32(gi.bf16_bits(A.astype(np.float32)))
    assert np.array_equal(sl[0], Af[:, cols]), "one-hot: y != A[:, j]"


def test_timeout_reports_missing_peer_and_skips_out():
    """Peer 3 withheld (its flags stay 0): every tile's wait expires after the
    (short) bound; status names tile 0 / peer 3; out stays unwritten; the own
    slot is still published."""
    _say("[protocol] timeout, whole peer withheld")
    W, rank = 4, 1
    d = gi.make_shard_inputs(W, 64, 256, 2, seed=10, rank=rank)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        r = Run(d["A"], d["x"], d["slots"].copy(), rank, published_mask=all_but(W, rank) & ~(1 << 3))
        try:
            r.call()
            out, sl, flags, status = r.results()
        finally:
            r.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)
    before = oracle.pad_after_reset(W, 64, all_but(W, rank) & ~(1 << 3))
    tiles, first = oracle.expected_timeouts(before, rank)
    assert status == (gsa.GSA_ETIMEOUT, first[0], first[1])
    assert np.isnan(out).all(), "timed-out tiles must not write out"
    y64, abs64, _ = oracle.load().gemv_allreduce(d["A"], d["x"], d["slots"], rank)
    assert np.all(np.abs(sl[rank] - y64) <= oracle.bound(abs64)), "own slot must be published"
    assert np.array_equal(flags, oracle.pad_after_calls(before, rank, 1))


@pytest.mark.parametrize("Ks,t_bad,B", [
    (128, 3, 3),     # short rows: 4-row workgroups, one flag tile each
    (1024, 6, 3),    # middle rows: 16-row workgroups of 4 waves; the third flag tile of the second
    (3200, 5, 3),    # long rows: 32-row workgroups; flag tile 5 is the sixth of its workgroup
    (3200, 13, 3),   # long rows: a flag tile of the second (ragged) 32-row workgroup
    (128, 19, 3),    # the last flag tile
    (2048, 5, 16),   # MFMA, A staged through LDS: 32-row workgroups
    (2048, 13, 12),  # the same, a flag tile of the second (ragged) workgroup
])
def test_timeout_single_tile(Ks, t_bad, B):
    """One flag word of peer 2 overwritten with 0 from the host: only the rows
    of that flag tile stay unwritten, whatever the workgroup size; every other
    row is correct."""
    _say(f"[protocol] timeout, one flag tile withheld, Ks={Ks} t={t_bad} B={B}")
    W, rank, N = 4, 0, 80
    d = gi.make_shard_inputs(W, N, Ks, B, seed=11, rank=rank)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        r = Run(d["A"], d["x"], d["slots"].copy(), rank)
        try:
            pad = r.buf.pad_view()
            pad[gsa.GSA_PAD_HEADER_WORDS + 2 * r.buf.row_stride + gsa.flag_word(t_bad)] = 0
            torch.cuda.synchronize()
            r.call()
            out, sl, flags, status = r.results()
        finally:
            r.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)
    assert status == (gsa.GSA_ETIMEOUT, t_bad, 2)
    ft = oracle.FLAG_TILE_ROWS
    rows = slice(ft * t_bad, min(N, ft * (t_bad + 1)))
    assert np.isnan(out[rows]).all()
    mask = np.ones(N, bool)
    mask[rows] = False
    y64, abs64, out64 = oracle.load().gemv_allreduce(d["A"], d["x"], d["slots"], rank)
    bnd = oracle.bound(abs64)
    assert np.all(np.abs(out[mask] - out64[mask]) <= bnd[mask])
    assert np.all(np.abs(sl[rank] - y64) <= bnd)


def test_own_row_marked_published_is_rejected_on_device():
    """Calling as a rank whose flag row is marked published: status
    GSA_ESTATE, nothing written, flags unchanged."""
    _say("[protocol] bad own row")
    W, rank = 2, 0
    d = gi.make_shard_inputs(W, 48, 64, 1, seed=12, rank=rank)
    r = Run(d["A"], d["x"], d["slots"].copy(), rank, published_mask=0b11)
    try:
        r.call()
        out, sl, flags, status = r.results()
    finally:
        r.close()
    assert status[0] == gsa.GSA_ESTATE and status[1] == 0
    assert np.isnan(out).all() and np.isnan(sl[rank]).all()
    assert np.array_equal(flags, oracle.pad_after_reset(W, 48, 0b11))


def test_reset_clears_status_and_flags():
    _say("[protocol] reset")
    W, rank = 2, 1
    d = gi.make_shard_inputs(W, 32, 64, 1, seed=13, rank=rank)
    r = Run(d["A"], d["x"], d["slots"].copy(), rank, published_mask=0b11)
    try:
        r.call()
        assert r.results()[3][0] == gsa.GSA_ESTATE
        r.buf.reset(all_but(W, rank))
        r.call()
        out, sl, flags, status = r.results()
        assert status == (gsa.GSA_OK, -1, -1)
        check_against_oracle(d["A"], d["x"], d["slots"], rank, out, sl, "after reset")
        assert np.array_equal(flags, oracle.pad_after_calls(oracle.pad_after_reset(W, 32, 0b01), 1, 1))
    finally:
        r.close()


def test_graph_replays_match_eager():
    """Calls captured in a HIP graph: every replay's output equals the eager
    result bit for bit, with eager work and syncs between replays."""
    _say("[protocol] graph replays")
    d = gi.make_inputs("c3b4", seed=14)
    r = Run(d["A"], d["x"], d["slots"].copy(), 0)
    try:
        r.call()
        eager, _, _, _ = r.results()
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                r.call()
        for i in range(4):
            r.out.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            out, sl, flags, status = r.results()
            assert status == (gsa.GSA_OK, -1, -1)
            assert np.array_equal(_bits(out), _bits(eager)), f"replay {i} differs"
            _ = torch.ones(8, device="cuda").sum().item()  # eager work between replays
        assert (flags[0] == 5).all()  # one eager call + four replays
    finally:
        r.close()
