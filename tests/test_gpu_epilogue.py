"""GPU parity of the fused epilogue (bias, RMSNorm over rows, fp32 or bf16 y)
through the C ABI (gsa_gemv_allreduce_rmsnorm), against the CPU oracle.

Per call: `out` meets the usual bar (bound vs fp64, bit-exact rank-order
fold of the slots read back); inv_rms is within an a-priori bound of the fp64
value computed from z = fl32(out + bias); y is bit-identical to the fp32
evaluation (z * inv) * w given the kernel's inv_rms (and its bf16 rounding).
"""
import math
import sys

import numpy as np
import pytest
import torch

import gemv_shot_all_amd as gsa
import gsa_inputs as gi
import oracle
from tests.gpu_util import Run, all_but, check_against_oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def inv_rel_bound(N):
    """Relative bound on the kernel's fp32 1/rms: the sum of squares runs 16
    sequential adds per tile, then at most ceil(T/16) per lane of the fold
    (a lane takes every (nt/P)-th record, nt >= 256 threads, P <= 16 lanes
    per record), a lane tree of at most 6 levels and at most 8 wave sums in
    order (depth d), after one rounding per square; then a division by N,
    the +eps, the square root (which halves the relative error) and the
    reciprocal each round once."""
    T = (N + 15) // 16
    d = 16 + math.ceil(T / 16) + 6 + 8
    return ((d + 3) / 2 + 3) * U


class EpiRun:
    def __init__(self, d, rank=None, bias=True, weight=True, eps=1e-5, y_dtype=torch.float32,
                 seed=0, published_mask=None):
        self.d = d
        self.rank = d["rank"] if rank is None else rank
        self.slots_in = d["slots"].copy()
        self.r = Run(d["A"], d["x"], self.slots_in, self.rank, published_mask)
        N, B = self.r.N, self.r.B
        rng = np.random.default_rng(seed + 77)
        self.bias = rng.normal(0, 0.5, N).astype(np.float32) if bias else None
        self.w = rng.normal(1, 0.1, N).astype(np.float32) if weight else None
        self.eps = eps
        self.bias_t = None if self.bias is None else torch.from_numpy(self.bias).cuda()
        self.w_t = None if self.w is None else torch.from_numpy(self.w).cuda()
        self.y = torch.full((N, B), float("nan"), dtype=y_dtype, device="cuda")
        self.inv = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
        self.ep = gsa.make_epilogue(self.y, self.bias_t, self.w_t, eps, self.inv)

    def call(self):
        r = self.r
        gsa.gsa_gemv_allreduce_rmsnorm(r.A, r.x, r.buf.slots, r.buf.pad, r.out, r.W, self.rank,
                                       r.N, r.K, r.B, self.ep)

    def results(self):
        out, slots, flags, status = self.r.results()
        y = self.y.cpu()
        y = (y.view(torch.int16).numpy().view(np.uint16) if self.y.dtype == torch.bfloat16
             else y.numpy())
        hdr = self.r.buf.pad_view()[:gsa.GSA_PAD_HEADER_WORDS].cpu().numpy()
        return out, slots, y, self.inv.cpu().numpy(), status, hdr

    def close(self):
        self.r.close()


def check_epilogue(er, out, slots_out, y, inv, what):
    d = er.d
    check_against_oracle(d["A"], d["x"], er.slots_in, er.rank, out, slots_out, what)
    o = oracle.load()
    z, inv64, y64 = o.bias_rmsnorm(out, er.bias, er.w, er.eps)
    rel = inv_rel_bound(out.shape[0])
    err = np.abs(inv.astype(np.float64) - inv64) / inv64
    assert np.all(err <= rel), f"{what}: inv_rms rel err {err.max():.3g} > {rel:.3g}"
    y32, ybf = o.scale_f32(z, inv, er.w)
    if y.dtype == np.uint16:
        assert np.array_equal(y, ybf), f"{what}: bf16 y differs from RNE of (z*inv)*w"
    else:
        assert np.array_equal(y.view(np.uint32), y32.view(np.uint32)), (
            f"{what}: y differs from (z*inv)*w given the kernel's inv_rms")
        # and close to the fp64 value
        lim = np.abs(y64) * (rel + 3 * U) + 1e-30
        assert np.all(np.abs(y.astype(np.float64) - y64) <= lim), f"{what}: y vs fp64"


def run_epi_and_check(d, what, **kw):
    er = EpiRun(d, **kw)
    try:
        er.call()
        out, sl, y, inv, status, hdr = er.results()
    finally:
        er.close()
    assert status == (gsa.GSA_OK, -1, -1), f"{what}: status {status}"
    check_epilogue(er, out, sl, y, inv, what)


@pytest.mark.parametrize("cfg", ["c1", "c2", "c3b4", "c4", "c5"])
@pytest.mark.parametrize("ydt", ["f32", "bf16"])
def test_config_epilogue(cfg, ydt):
    _say(f"[epilogue] config {cfg} y={ydt}")
    d = gi.make_inputs(cfg, seed=0, rank=0)
    run_epi_and_check(d, f"{cfg}/{ydt}",
                      y_dtype=torch.float32 if ydt == "f32" else torch.bfloat16)


EDGE = [
    # (W, N, Ks, B, rank, bias, weight, eps)
    (2, 1000, 512, 1, 1, True, True, 1e-6),      # ragged N
    (8, 17, 512, 3, 7, True, False, 1e-5),       # 2 tiles, the second with one row
    (1, 1, 8, 1, 0, False, False, 1e-3),         # one row
    # calls of at most 64 records x columns, where every waiting workgroup
    # folds the records itself, and the first call past that bound
    (4, 256, 512, 4, 2, True, True, 1e-5),       # 16 tiles x 4 columns: 64
    (2, 100, 256, 2, 0, True, False, 1e-5),      # 7 tiles x 2, the last ragged
    (8, 64 * 16, 512, 1, 3, False, True, 1e-5),  # 64 tiles x 1
    (8, 65 * 16, 512, 1, 3, True, True, 1e-5),   # 65 tiles: one workgroup folds
    (4, 50, 2048, 9, 3, False, True, 0.0),       # MFMA, ragged, eps = 0
    (4, 4000, 256, 16, 1, True, True, 1e-5),     # MFMA, 250 tiles: several per fold lane
    (8, 8192 + 16 * 65, 64, 2, 5, True, True, 1e-5),  # 577 tiles, short rows
    (2, 65536, 64, 1, 0, True, True, 1e-5),     # 4096 tiles: more than fit at once
    # 2048 tiles of 4 columns: more than fit at once, so tiles that finish
    # early leave their rows to the folding workgroup
    (2, 2048 * 16 - 5, 512, 4, 1, True, True, 1e-5),
    (2, 16 * 6000 + 5, 64, 3, 1, True, False, 1e-4),  # 6001 tiles, ragged
]


@pytest.mark.parametrize("W,N,Ks,B,rank,bias,weight,eps", EDGE)
def test_edge_epilogue(W, N, Ks, B, rank, bias, weight, eps):
    _say(f"[epilogue] edge W={W} N={N} Ks={Ks} B={B} bias={bias} weight={weight} eps={eps}")
    d = gi.make_shard_inputs(W, N, Ks, B, sigma=0.02, seed=3, cfg_id=3000 + N + B, rank=rank)
    run_epi_and_check(d, f"W={W} N={N} Ks={Ks} B={B}", bias=bias, weight=weight, eps=eps)


@pytest.mark.parametrize("cfg", ["c1", "c2"])
def test_repeats_bit_identical_and_mixed_with_plain_calls(cfg):
    """Three epilogue calls with plain calls in between (which leave the
    epilogue's counts alone): y and inv_rms are right and bit-identical every
    time.  (On these shapes the plain call runs 4-row workgroups and the
    epilogue call 16-row ones, so their partial sums may round differently:
    each call's results are checked right after it.)  c1 has 64 records a
    call, so every waiting workgroup folds them; c2 256, folded by one."""
    _say(f"[epilogue] repeats {cfg}")
    d = gi.make_inputs(cfg, seed=4, rank=0)
    er = EpiRun(d, seed=4)
    try:
        ys, invs = [], []
        for i in range(3):
            er.call()
            out, sl, y, inv, status, hdr = er.results()
            assert status == (gsa.GSA_OK, -1, -1)
            check_epilogue(er, out, sl, y, inv, f"repeat {i}")
            ys.append(y.copy())
            invs.append(inv.copy())
            er.r.out.fill_(float("nan"))
            er.r.call()  # a plain call on the same buffer
            out, sl, _, status = er.r.results()
            assert status == (gsa.GSA_OK, -1, -1)
            check_against_oracle(d["A"], d["x"], er.slots_in, 0, out, sl, f"plain {i}")
    finally:
        er.close()
    for i in range(1, 3):
        assert np.array_equal(ys[i].view(np.uint32), ys[0].view(np.uint32))
        assert np.array_equal(invs[i].view(np.uint32), invs[0].view(np.uint32))


def test_timeout_poisons_y_then_recovers():
    """A withheld peer: the waits expire, y and inv_rms come out NaN (every
    tile still publishes its sums, so nothing hangs); after a reset with the
    peer published the next calls are correct."""
    _say("[epilogue] timeout")
    W, rank = 4, 1
    d = gi.make_shard_inputs(W, 64, 256, 2, seed=12, rank=rank)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        er = EpiRun(d, rank=rank, published_mask=all_but(W, rank) & ~(1 << 2))
        try:
            er.call()
            out, sl, y, inv, status, hdr = er.results()
            assert status[0] == gsa.GSA_ETIMEOUT
            assert np.isnan(y).all() and np.isnan(inv).all(), "a failed call must poison y"
            er.r.buf.reset(all_but(W, rank))
            er.y.fill_(float("nan"))
            er.r.out.fill_(float("nan"))
            er.call()
            out, sl, y, inv, status, hdr = er.results()
            assert status == (gsa.GSA_OK, -1, -1)
            check_epilogue(er, out, sl, y, inv, "after recovery")
            er.y.fill_(float("nan"))
            er.call()
            out, sl, y, inv, status, hdr = er.results()
            assert status == (gsa.GSA_OK, -1, -1)
            check_epilogue(er, out, sl, y, inv, "second call after recovery")
        finally:
            er.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)


@pytest.mark.parametrize("cfg", ["c1", "c3b4"])
def test_graph_replays_match_eager(cfg):
    """Calls captured in a HIP graph (no host-held state: the epilogue's
    counts only grow): every replay gives the eager result, bit for bit."""
    _say(f"[epilogue] graph replays {cfg}")
    d = gi.make_inputs(cfg, seed=5, rank=0)
    er = EpiRun(d, seed=5, y_dtype=torch.bfloat16)
    try:
        er.call()
        out0, sl0, y0, inv0, status, hdr = er.results()
        check_epilogue(er, out0, sl0, y0, inv0, "eager")
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for _ in range(3):
                    er.call()
        for rep in range(3):
            er.y.fill_(float("nan"))
            g.replay()
            torch.cuda.synchronize()
            out, sl, y, inv, status, hdr = er.results()
            assert status == (gsa.GSA_OK, -1, -1)
            assert np.array_equal(y, y0) and np.array_equal(inv.view(np.uint32),
                                                            inv0.view(np.uint32)), f"replay {rep}"
    finally:
        er.close()


@pytest.mark.parametrize("Ks", [256, 6400])
def test_plain_and_epilogue_calls_share_a_buffer(Ks):
    """Plain calls (4-row workgroups on short rows) and epilogue calls (16-row
    workgroups) alternate on one buffer: every call raises each 4-row flag
    tile once, so the epochs stay in step and every result is right."""
    _say(f"[epilogue] plain and epilogue calls on one buffer, Ks={Ks}")
    W, rank = 4, 2
    d = gi.make_shard_inputs(W, 200, Ks, 3, seed=21, rank=rank)
    er = EpiRun(d, rank=rank, seed=21)
    try:
        for i, kind in enumerate(["plain", "epilogue", "plain", "epilogue", "plain"]):
            er.r.out.fill_(float("nan"))
            if kind == "plain":
                er.r.call()
                out, sl, flags, status = er.r.results()
                assert status == (gsa.GSA_OK, -1, -1), (kind, i, status)
                check_against_oracle(d["A"], d["x"], er.slots_in, rank, out, sl, f"{kind} {i}")
            else:
                er.y.fill_(float("nan"))
                er.call()
                out, sl, y, inv, status, hdr = er.results()
                assert status == (gsa.GSA_OK, -1, -1), (kind, i, status)
                check_epilogue(er, out, sl, y, inv, f"{kind} {i}")
                flags = er.r.buf.flags()
            expect = oracle.pad_after_calls(oracle.pad_after_reset(W, 200, all_but(W, rank)),
                                            rank, i + 1)
            assert np.array_equal(flags, expect), f"{kind} {i}: flag state"
    finally:
        er.close()


def unfused_inv_rel_bound(N):
    """The same bound for gsa_bias_rmsnorm, whose sum runs ceil(N / 1024)
    sequential adds per thread, a 6-level lane butterfly and the 16 waves in
    order."""
    d = math.ceil(N / 1024) + 6 + 16
    return ((d + 3) / 2 + 3) * U


UNFUSED = [
    # (N, B, bias, weight, eps, y dtype)
    (4096, 1, True, True, 1e-5, torch.bfloat16),    # the o_proj shape
    (8192, 4, True, True, 1e-5, torch.float32),     # the 70B-class shape
    (8192, 16, True, True, 1e-5, torch.bfloat16),   # the skinny GEMM
    (1, 1, True, True, 1e-5, torch.float32),        # one row
    (1025, 3, False, True, 0.0, torch.float32),     # past one batch of rows, no bias, eps = 0
    (9000, 7, True, False, 1e-3, torch.float32),    # two batches, ragged, no weight
    (70000, 2, True, True, 1e-5, torch.bfloat16),   # many batches
]


@pytest.mark.parametrize("N,B,bias,weight,eps,y_dtype", UNFUSED)
def test_unfused_bias_rmsnorm(N, B, bias, weight, eps, y_dtype):
    """gsa_bias_rmsnorm on a seeded out: inv_rms within its bound of the fp64
    value, y bit-identical to (z * inv) * w given the kernel's inv_rms, and
    every call bit-identical."""
    _say(f"[epilogue] unfused N={N} B={B} bias={bias} weight={weight} eps={eps} y={y_dtype}")
    rng = np.random.default_rng(N * 31 + B)
    out = rng.normal(0, 1, (N, B)).astype(np.float32)
    b = rng.normal(0, 0.5, N).astype(np.float32) if bias else None
    w = rng.normal(1, 0.1, N).astype(np.float32) if weight else None
    out_t = torch.from_numpy(out).cuda()
    b_t = None if b is None else torch.from_numpy(b).cuda()
    w_t = None if w is None else torch.from_numpy(w).cuda()
    ys, invs = [], []
    for _ in range(2):
        y = torch.full((N, B), float("nan"), dtype=y_dtype, device="cuda")
        inv = torch.full((B,), float("nan"), dtype=torch.float32, device="cuda")
        gsa.gsa_bias_rmsnorm(out_t, N, B, gsa.make_epilogue(y, b_t, w_t, eps, inv))
        torch.cuda.synchronize()
        yc = y.cpu()
        ys.append(yc.view(torch.int16).numpy().view(np.uint16) if y_dtype == torch.bfloat16
                  else yc.numpy())
        invs.append(inv.cpu().numpy())
    assert np.array_equal(ys[0].view(np.uint8), ys[1].view(np.uint8))
    assert np.array_equal(invs[0].view(np.uint32), invs[1].view(np.uint32))
    o = oracle.load()
    z, inv64, y64 = o.bias_rmsnorm(out, b, w, eps)
    rel = unfused_inv_rel_bound(N)
    err = np.abs(invs[0].astype(np.float64) - inv64) / inv64
    assert np.all(err <= rel), f"inv_rms rel err {err.max():.3g} > {rel:.3g}"
    y32, ybf = o.scale_f32(z, invs[0], w)
    if y_dtype == torch.bfloat16:
        assert np.array_equal(ys[0], ybf)
    else:
        assert np.array_equal(ys[0].view(np.uint32), y32.view(np.uint32))


def test_plain_call_then_unfused_matches_fused_definition():
    """The unfused form of the epilogue on the o_proj shape: a plain call,
    then gsa_bias_rmsnorm on its out (same stream); out meets the usual bar
    and y the epilogue's."""
    d = gi.make_inputs("c2", seed=0, rank=0)
    er = EpiRun(d, y_dtype=torch.bfloat16)
    try:
        r = er.r
        gsa.gsa_gemv_allreduce(r.A, r.x, r.buf.slots, r.buf.pad, r.out, r.W, er.rank, r.N, r.K,
                               r.B)
        gsa.gsa_bias_rmsnorm(r.out, r.N, r.B, er.ep)
        out, sl, y, inv, status, hdr = er.results()
    finally:
        er.close()
    assert status == (gsa.GSA_OK, -1, -1)
    check_against_oracle(d["A"], d["x"], er.slots_in, er.rank, out, sl, "c2 plain")
    o = oracle.load()
    z, inv64, y64 = o.bias_rmsnorm(out, er.bias, er.w, er.eps)
    rel = unfused_inv_rel_bound(out.shape[0])
    assert np.all(np.abs(inv.astype(np.float64) - inv64) / inv64 <= rel)
    y32, ybf = o.scale_f32(z, inv, er.w)
    assert np.array_equal(y, ybf)
