"""Helpers for the GPU tests: run the HIP path through the C ABI on seeded
inputs and compare with the CPU oracle."""
import numpy as np
import torch

import gemv_shot_all_amd as gsa
import oracle

NAN_BITS = 0x7FC00000


def to_dev(a):
    """numpy -> cuda tensor (uint16 goes as int16 bits)."""
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def all_but(W, rank):
    return ((1 << W) - 1) & ~(1 << rank)


class Run:
    """One prepared call: device inputs, a symmetric buffer and an output."""

    def __init__(self, A, x, slots, rank, published_mask=None):
        self.A_np, self.x_np, self.slots_np = A, x, slots
        self.W, self.N, self.B = slots.shape
        self.Ks = A.shape[1]
        self.K = self.Ks * self.W
        self.rank = rank
        self.A = to_dev(A)
        self.x = to_dev(x)
        self.buf = gsa.SymmBuffer(self.W, self.N, self.B)
        self.buf.slots_view().copy_(torch.from_numpy(slots).cuda())
        self.out = torch.full((self.N, self.B), float("nan"), dtype=torch.float32, device="cuda")
        mask = all_but(self.W, rank) if published_mask is None else published_mask
        self.buf.reset(mask)

    def call(self, rank=None, A=None, x=None):
        gsa.gsa_gemv_allreduce(self.A if A is None else A, self.x if x is None else x,
                               self.buf.slots, self.buf.pad, self.out, self.W,
                               self.rank if rank is None else rank, self.N, self.K, self.B)

    def results(self):
        torch.cuda.synchronize()
        return (self.out.cpu().numpy(), self.buf.slots_view().cpu().numpy(),
                self.buf.flags(), self.buf.status())

    def close(self):
        self.buf.close()


def check_against_oracle(A, x, slots_in, rank, out, slots_out, what=""):
    """The parity bar: published slot and out within the error bound of the
    fp64 oracle, out bit-identical to the fp32 rank-order fold of the slots
    as read back, peer slots untouched."""
    y64, abs64, out64 = oracle.load().gemv_allreduce(A, x, slots_in, rank)
    bnd = oracle.bound(abs64)
    W = slots_in.shape[0]
    y = slots_out[rank]
    err_y = np.abs(y.astype(np.float64) - y64)
    assert np.all(err_y <= bnd), (
        f"{what}: slot[rank] off: max err/bound {np.max(err_y / bnd):.3g} at "
        f"{np.unravel_index(np.argmax(err_y / bnd), y.shape)}")
    err_o = np.abs(out.astype(np.float64) - out64)
    assert np.all(err_o <= bnd), (
        f"{what}: out off: max err/bound {np.max(err_o / bnd):.3g}")
    fold = oracle.load().fold_f32(slots_out)
    assert np.array_equal(out.view(np.uint32), fold.view(np.uint32)), (
        f"{what}: out is not the rank-order fp32 fold of the slots")
    for r in range(W):
        if r != rank:
            assert np.array_equal(slots_out[r].view(np.uint32), slots_in[r].view(np.uint32)), (
                f"{what}: peer slot {r} modified")
    return float(np.max(err_o / bnd)), float(np.max(err_y / bnd))


def run_and_check(d, rank=None, what=""):
    rank = d["rank"] if rank is None else rank
    slots = d["slots"].copy()
    r = Run(d["A"], d["x"], slots, rank)
    try:
        r.call()
        out, slots_out, flags, status = r.results()
    finally:
        r.close()
    assert status == (gsa.GSA_OK, -1, -1), f"{what}: status {status}"
    ratio = check_against_oracle(d["A"], d["x"], slots, rank, out, slots_out, what)
    W = slots.shape[0]
    expect = oracle.pad_after_calls(oracle.pad_after_reset(W, slots.shape[1], all_but(W, rank)),
                                    rank, 1)
    assert np.array_equal(flags, expect), f"{what}: flag state"
    return ratio
