"""bf16 slots and bf16 out of the fused call (gsa_gemv_allreduce_dtype)
against the oracle on the GPU (needs an MI355X).

The reading ("PyTorch Symmetric Memory" documentation, higher-precision
reduction section): bf16 values in, fp32 accumulation, bf16 out.  A buffer
with bf16 slots publishes y rounded to bf16 and the one-shot sum widens every
slot value and adds in fp32; a bf16 out is the fp32 sum rounded to nearest,
ties to even.  Parity bar, every call:
  * the published own value within the fp32 bound of the fp64 product, plus
    half a bf16 unit in the last place for bf16 slots (oracle.bound_bf16);
  * out bit-identical to the oracle's fp32 fold of the slots as read back
    (fold_bf16 for bf16 slots, fold_f32 otherwise), rounded to bf16 by the
    oracle for a bf16 out;
  * out within the derived tolerance of the fp64 value (see _out_tolerance);
  * peer slots untouched, flags as the protocol predicts."""
import sys

import numpy as np
import pytest
import torch

import gemv_shot_all_amd as gsa
import gsa_inputs as gi
import oracle
from tests.gpu_util import all_but, to_dev

pytestmark = pytest.mark.gpu

F32, BF16 = gsa.GSA_DTYPE_F32, gsa.GSA_DTYPE_BF16
NAN_BF16 = 0x7FC0


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


def _widen(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


class DRun:
    """One prepared call with element types: device inputs, a buffer whose
    peer slots hold the seeded values (rounded to bf16 for bf16 slots), and a
    NaN-filled out of out_dtype."""

    def __init__(self, d, rank, slot_dtype, out_dtype, published_mask=None):
        self.d, self.rank = d, rank
        self.W, self.N, self.B = d["slots"].shape
        self.K = d["A"].shape[1] * self.W
        self.slot_dtype, self.out_dtype = slot_dtype, out_dtype
        if slot_dtype == BF16:
            # peers rounded to bf16 (like A and x); the own slot a NaN sentinel
            self.slots_in = np.full(d["slots"].shape, NAN_BF16, np.uint16)
            for p in range(self.W):
                if p != rank:
                    self.slots_in[p] = gi.bf16_bits(d["slots"][p])
            peer_vals = torch.from_numpy(self.slots_in.view(np.int16)).cuda()
        else:
            self.slots_in = d["slots"].copy()
            peer_vals = torch.from_numpy(self.slots_in).cuda()
        self.A, self.x = to_dev(d["A"]), to_dev(d["x"])
        self.buf = gsa.SymmBuffer(self.W, self.N, self.B, slot_dtype)
        self.buf.slots_view().copy_(peer_vals)
        if out_dtype == BF16:
            self.out = torch.full((self.N, self.B), NAN_BF16, dtype=torch.int16, device="cuda")
        else:
            self.out = torch.full((self.N, self.B), float("nan"), dtype=torch.float32,
                                  device="cuda")
        self.buf.reset(all_but(self.W, rank) if published_mask is None else published_mask)

    def call(self):
        gsa.gsa_gemv_allreduce_dtype(self.A, self.x, self.buf.slots, self.buf.pad, self.out,
                                     self.out_dtype, self.W, self.rank, self.N, self.K, self.B)

    def results(self):
        torch.cuda.synchronize()
        out = self.out.cpu().numpy()
        slots = self.buf.slots_view().cpu().numpy()
        if self.out_dtype == BF16:
            out = out.view(np.uint16)
        if self.slot_dtype == BF16:
            slots = slots.view(np.uint16)
        return out, slots, self.buf.flags(), self.buf.status()

    def close(self):
        self.buf.close()


def _out_tolerance(own_err, slot_vals, out64, out_bf16):
    """|out - out64| allowed: the own term's error (the peers are exact
    inputs), plus the fp32 fold's rounding -- each of its W - 1 adds rounds
    to nearest, at most 2^-24 of a partial sum, itself at most sum_r |s_r| --
    plus, for a bf16 out, half a bf16 unit in the last place, at most 2^-8 of
    the value."""
    W = slot_vals.shape[0]
    mag = np.sum(np.abs(slot_vals.astype(np.float64)), axis=0)
    tol = own_err + (W - 1) * 2.0 ** -24 * mag
    if out_bf16:
        tol = tol + 2.0 ** -8 * (np.abs(out64) + tol)
    return tol


def check_dtype_call(r, out, slots_out, flags, status, what):
    o = oracle.load()
    d, rank, W = r.d, r.rank, r.W
    assert status == (gsa.GSA_OK, -1, -1), f"{what}: status {status}"
    peers_f32 = _widen(r.slots_in) if r.slot_dtype == BF16 else r.slots_in
    y64, abs64, out64 = o.gemv_allreduce(d["A"], d["x"], peers_f32, rank)
    # the published own value
    if r.slot_dtype == BF16:
        y = _widen(slots_out[rank]).astype(np.float64)
        own_bound = oracle.bound_bf16(abs64, y64)
    else:
        y = slots_out[rank].astype(np.float64)
        own_bound = oracle.bound(abs64)
    err = np.abs(y - y64)
    assert np.all(err <= own_bound), (
        f"{what}: published value off, max err/bound {np.max(err / own_bound):.3g}")
    # out: the fold of the slots as read back, bit for bit
    if r.slot_dtype == BF16:
        fold = o.fold_bf16(slots_out)
        vals = _widen(slots_out)
    else:
        fold = o.fold_f32(slots_out)
        vals = slots_out
    if r.out_dtype == BF16:
        want = o.to_bf16(fold)
        assert np.array_equal(out, want), (
            f"{what}: bf16 out is not the rounded fp32 fold of the slots "
            f"({int(np.sum(out != want))} elements)")
        outv = _widen(out).astype(np.float64)
    else:
        assert np.array_equal(out.view(np.uint32), fold.view(np.uint32)), (
            f"{what}: out is not the fp32 fold of the slots")
        outv = out.astype(np.float64)
    tol = _out_tolerance(own_bound, vals, out64, r.out_dtype == BF16)
    e = np.abs(outv - out64)
    assert np.all(e <= tol), f"{what}: out off, max err/tol {np.max(e / tol):.3g}"
    # peers untouched, flags as predicted
    for p in range(W):
        if p != rank:
            assert np.array_equal(np.asarray(slots_out[p]).view(np.uint8),
                                  np.asarray(r.slots_in[p]).view(np.uint8)), (
                f"{what}: peer slot {p} modified")
    expect = oracle.pad_after_calls(oracle.pad_after_reset(W, r.N, all_but(W, rank)), rank, 1)
    assert np.array_equal(flags, expect), f"{what}: flag state"
    return float(np.max(e / tol))


DTYPES = [(BF16, BF16), (BF16, F32), (F32, BF16)]
_NAMES = {F32: "f32", BF16: "bf16"}


def _ids(p):
    return f"slots_{_NAMES[p[0]]}-out_{_NAMES[p[1]]}"


@pytest.mark.parametrize("dts", DTYPES, ids=_ids)
@pytest.mark.parametrize("cfg", list(gi.CONFIGS))
def test_config_dtype_parity(cfg, dts):
    _say(f"[dtype] {cfg} {_ids(dts)}")
    d = gi.make_inputs(cfg, seed=0, rank=0)
    r = DRun(d, 0, *dts)
    try:
        r.call()
        res = r.results()
    finally:
        r.close()
    ratio = check_dtype_call(r, *res, what=f"{cfg} {_ids(dts)}")
    _say(f"[dtype] {cfg} {_ids(dts)}: max err/tol {ratio:.3g}")


EDGE = [
    # (W, N, Ks, B, rank): one case per kernel tier
    (2, 1000, 512, 1, 1),     # 4-row tiles, ragged N
    (4, 123, 512, 8, 2),      # 4-row tiles, B = 8, the last tile 3 rows
    (8, 100, 1792, 8, 3),     # 16-row middle tier, B = 8
    (4, 70, 3584, 4, 1),      # 32-row long tier (unrolled), ragged N
    (2, 33, 5000, 5, 0),      # long tier, masked rows, B = 5
    (4, 50, 2048, 9, 3),      # MFMA, B = 9, ragged N
    (2, 32, 8192, 16, 1),     # MFMA, x read from memory
    (1, 70, 256, 16, 0),      # W = 1
]


@pytest.mark.parametrize("dts", DTYPES, ids=_ids)
@pytest.mark.parametrize("W,N,Ks,B,rank", EDGE)
def test_edge_dtype_parity(W, N, Ks, B, rank, dts):
    _say(f"[dtype] edge W={W} N={N} Ks={Ks} B={B} rank={rank} {_ids(dts)}")
    d = gi.make_shard_inputs(W, N, Ks, B, sigma=0.02, seed=5, cfg_id=3000 + N + Ks + B,
                             rank=rank)
    r = DRun(d, rank, *dts)
    try:
        r.call()
        res = r.results()
    finally:
        r.close()
    check_dtype_call(r, *res, what=f"W={W} N={N} Ks={Ks} B={B} {_ids(dts)}")


def test_dtype_f32_equals_plain_call():
    """fp32 slots and fp32 out through the typed entry point: the same bits as
    gsa_gemv_allreduce."""
    _say("[dtype] f32/f32 equals the plain call")
    d = gi.make_inputs("c3b4", seed=2, rank=0)
    r = DRun(d, 0, F32, F32)
    try:
        r.call()
        out_t, sl_t, _, st = r.results()
        r.buf.reset(all_but(r.W, 0))
        r.out.fill_(float("nan"))
        gsa.gsa_gemv_allreduce(r.A, r.x, r.buf.slots, r.buf.pad, r.out, r.W, 0, r.N, r.K, r.B)
        out_p, sl_p, _, st2 = r.results()
    finally:
        r.close()
    assert st == st2 == (gsa.GSA_OK, -1, -1)
    assert np.array_equal(out_t.view(np.uint32), out_p.view(np.uint32))
    assert np.array_equal(sl_t.view(np.uint32), sl_p.view(np.uint32))


def test_dtype_repeats_bit_identical():
    _say("[dtype] repeats")
    d = gi.make_inputs("c4", seed=3, rank=0)
    r = DRun(d, 0, BF16, BF16)
    try:
        r.call()
        out0, sl0, _, _ = r.results()
        for i in range(1, 20):
            r.out.fill_(NAN_BF16)
            r.call()
            out, sl, flags, status = r.results()
            assert np.array_equal(out, out0) and np.array_equal(sl, sl0), f"call {i} differs"
        assert status == (gsa.GSA_OK, -1, -1) and (flags[0] == 20).all()
    finally:
        r.close()


def test_bf16_slots_withheld_peer_times_out():
    """bf16 slots, one peer withheld: the late path waits (bounded), reports
    the first (flag tile, peer), leaves out unwritten and still publishes."""
    _say("[dtype] bf16 slots, withheld peer")
    W, rank = 4, 1
    d = gi.make_shard_inputs(W, 64, 3584, 2, seed=10, rank=rank)
    mask = all_but(W, rank) & ~(1 << 3)
    gsa.gsa_set_wait_timeout_us(200)
    try:
        r = DRun(d, rank, BF16, BF16, published_mask=mask)
        try:
            r.call()
            out, sl, flags, status = r.results()
        finally:
            r.close()
    finally:
        gsa.gsa_set_wait_timeout_us(100000)
    before = oracle.pad_after_reset(W, 64, mask)
    _, first = oracle.expected_timeouts(before, rank)
    assert status == (gsa.GSA_ETIMEOUT, first[0], first[1])
    assert (out == NAN_BF16).all(), "timed-out tiles must not write out"
    y64, abs64, _ = oracle.load().gemv_allreduce(d["A"], d["x"], _widen(r.slots_in), rank)
    y = _widen(sl[rank]).astype(np.float64)
    assert np.all(np.abs(y - y64) <= oracle.bound_bf16(abs64, y64))


def test_bf16_slot_buffer_rejected_by_other_calls():
    """The two-shot and epilogue calls, and the plain call, take fp32 slots
    only: a bf16-slot buffer is rejected before any launch."""
    W, N, B, Ks = 2, 32, 1, 64
    d = gi.make_shard_inputs(W, N, Ks, B, seed=1, rank=0)
    A, x = to_dev(d["A"]), to_dev(d["x"])
    out = torch.zeros((N, B), dtype=torch.float32, device="cuda")
    with gsa.SymmBuffer(W, N, B, BF16) as buf:
        buf.reset(all_but(W, 0))
        with pytest.raises(gsa.GsaError) as e:
            gsa.gsa_gemv_allreduce(A, x, buf.slots, buf.pad, out, W, 0, N, Ks * W, B)
        assert e.value.code == gsa.GSA_EINVAL
        with pytest.raises(gsa.GsaError) as e:
            gsa.gsa_gemv_allreduce_two_shot(A, x, buf.slots, buf.pad, buf.gathered, out, W, 0,
                                            N, Ks * W, B)
        assert e.value.code == gsa.GSA_EINVAL
        y = torch.zeros((N, B), dtype=torch.float32, device="cuda")
        with pytest.raises(gsa.GsaError) as e:
            gsa.gsa_gemv_allreduce_rmsnorm(A, x, buf.slots, buf.pad, out, W, 0, N, Ks * W, B,
                                           gsa.make_epilogue(y))
        assert e.value.code == gsa.GSA_EINVAL
        with pytest.raises(gsa.GsaError) as e:
            gsa.gsa_gemv_allreduce_dtype(A, x, buf.slots, buf.pad, out, 7, W, 0, N, Ks * W, B)
        assert e.value.code == gsa.GSA_EINVAL
