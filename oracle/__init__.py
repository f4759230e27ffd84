"""CPU oracle for one rank's fused GEMV + AllReduce (and the MoE GEMM + combine).

TEST INFRASTRUCTURE.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  It shares no code with
the HIP library (`gemv_shot_all_amd`) and never imports it.

The arithmetic lives in `gsa_oracle.c` (plain C, fp64); this module loads it
with ctypes and adds numpy-facing wrappers plus a model of the signal-pad
protocol state.  Sources followed (restated, not quoted):

* fused GEMV + AllReduce operator -- "Overlapping Collective Communication
  with Dependent Computation ... GPU-Initiated Intra-Kernel Networking"
  (summary of "Optimizing Distributed ML Communication with Fused
  Computation-Collective Operations"), Abstract;
* row-parallel shard and one all-reduce at the end -- "Bay.Area.AI: Tensor and
  2D Parallelism", Megatron MLP segment;
* zero-initialised accumulator, every rank's buffer in rank order --
  "PyTorch Symmetric Memory" documentation, writing-your-own-kernel section
  (Triton one_shot_all_reduce_kernel);
* fp32 accumulation of bf16 inputs -- same documentation, higher-precision
  reduction section; read for the all-reduce itself: bf16 partials in the
  slots widened and summed in fp32, the sum handed back in bf16;
* bias then RMSNorm fused behind the all-reduce -- "PyTorch Symmetric Memory"
  talk, real-model example (RMSNorm itself: its textbook definition, the
  pages do not write it out); bf16 output of an fp32 accumulation -- the
  documentation's higher-precision reduction section;
* two-shot variant (reduce-scatter of an owned chunk, then all-gather) --
  the documentation's op reference of two_shot_all_reduce_;
* GEMM + All-to-All for mixture-of-experts -- the fused-operators page,
  Abstract; the expert-major dispatch layout and the combine that sends each
  segment back to its source rank at an offset it chose -- the
  documentation's op reference of all_to_all_vdev_2d and
  all_to_all_vdev_2d_offset;
* signal pad next to every symmetric allocation, sized by launched blocks
  times world size, indexed by block -- same documentation, the
  writing-your-own-kernel section and the set_signal_pad_size and
  multimem_all_reduce_ entries of the API and op reference.

Pins: every function here is checked against something other than itself in
tests/test_oracle_pins.py (numpy fp64 matmul on tiny shapes, closed forms,
hand-computed fp32 folds, shard-sum identity); tests/test_oracle_mutants.py
plants mistakes in a copy of the C source and checks that a pin fails.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)

# Protocol reading (the pages leave the granularity open): one flag per rank
# per flag tile of 4 output rows (all batch columns), so a rank's row of the
# pad holds ceil(N / 4) flags.  A simulated peer that has "published for every
# call" holds the all-ones word.
FLAG_TILE_ROWS = 4
FLAG_PUBLISHED = 0xFFFFFFFF

# The error bound every fp32 GPU result must meet against the fp64 value:
# |err| <= 1e-5 * sum_k |A[n,k] x[b,k]| + 1e-6.
BOUND_REL = 1e-5
BOUND_ABS = 1e-6


def _ptr(arr, ptype):
    return arr.ctypes.data_as(ptype)


class Oracle:
    """ctypes view of one build of the oracle library."""

    def __init__(self, path):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.gsa_oracle_gemv.argtypes = [_u16p, _u16p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int, _f64p, _f64p]
        lib.gsa_oracle_gemv.restype = ctypes.c_int
        lib.gsa_oracle_gemv_allreduce.argtypes = [
            _u16p, _u16p, _f32p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int, _f64p, _f64p, _f64p]
        lib.gsa_oracle_gemv_allreduce.restype = ctypes.c_int
        lib.gsa_oracle_fold_f32.argtypes = [_f32p, ctypes.c_int, ctypes.c_int64, _f32p]
        lib.gsa_oracle_fold_f32.restype = None
        lib.gsa_oracle_fold_bf16.argtypes = [_u16p, ctypes.c_int, ctypes.c_int64, _f32p]
        lib.gsa_oracle_fold_bf16.restype = None
        lib.gsa_oracle_f32_to_bf16.argtypes = [_f32p, ctypes.c_int64, _u16p]
        lib.gsa_oracle_f32_to_bf16.restype = None
        lib.gsa_oracle_bias_rmsnorm.argtypes = [_f32p, _f32p, _f32p, ctypes.c_double,
                                                ctypes.c_int64, ctypes.c_int, _f32p, _f64p,
                                                _f64p]
        lib.gsa_oracle_bias_rmsnorm.restype = ctypes.c_int
        lib.gsa_oracle_scale_f32.argtypes = [_f32p, _f32p, _f32p, ctypes.c_int64, ctypes.c_int,
                                             _f32p, _u16p]
        lib.gsa_oracle_scale_f32.restype = None
        lib.gsa_oracle_two_shot_chunk_rows.argtypes = [ctypes.c_int64, ctypes.c_int]
        lib.gsa_oracle_two_shot_chunk_rows.restype = ctypes.c_int64
        lib.gsa_oracle_two_shot.argtypes = [_f32p, _f32p, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int64, ctypes.c_int, _f32p, _f32p]
        lib.gsa_oracle_two_shot.restype = None
        _i32p = ctypes.POINTER(ctypes.c_int32)
        lib.gsa_oracle_moe_combine.argtypes = [
            _u16p, _u16p, _i32p, _i32p, _i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int64,
            ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, _f64p, _f64p,
            ctypes.POINTER(ctypes.c_uint8)]
        lib.gsa_oracle_moe_combine.restype = ctypes.c_int
        self._i32p = _i32p
        self._lib = lib

    def gemv(self, A, x):
        """fp64 y[n, b] = sum_k A[n, k] x[b, k] and sum_k |A[n, k] x[b, k]|.

        A: uint16 bf16 bits, N x Ks; x: uint16 bf16 bits, B x Ks.
        """
        A = np.ascontiguousarray(A, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        N, Ks = A.shape
        B, Ks2 = x.shape
        if Ks2 != Ks:
            raise ValueError("A and x disagree on the reduction length")
        y = np.empty((N, B), np.float64)
        a = np.empty((N, B), np.float64)
        rc = self._lib.gsa_oracle_gemv(_ptr(A, _u16p), _ptr(x, _u16p), N, Ks, B,
                                       _ptr(y, _f64p), _ptr(a, _f64p))
        if rc != 0:
            raise ValueError("oracle rejected the sizes")
        return y, a

    def gemv_allreduce(self, A, x, slots, rank):
        """One rank's call: (y64, abs64, out64), each N x B float64.

        slots: float32 W x N x B; row `rank` is ignored (the call publishes it).
        """
        A = np.ascontiguousarray(A, dtype=np.uint16)
        x = np.ascontiguousarray(x, dtype=np.uint16)
        slots = np.ascontiguousarray(slots, dtype=np.float32)
        N, Ks = A.shape
        B = x.shape[0]
        W = slots.shape[0]
        if x.shape[1] != Ks or slots.shape[1:] != (N, B):
            raise ValueError("shape mismatch")
        y = np.empty((N, B), np.float64)
        a = np.empty((N, B), np.float64)
        out = np.empty((N, B), np.float64)
        rc = self._lib.gsa_oracle_gemv_allreduce(
            _ptr(A, _u16p), _ptr(x, _u16p), _ptr(slots, _f32p), W, rank, N, Ks, B,
            _ptr(y, _f64p), _ptr(a, _f64p), _ptr(out, _f64p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return y, a, out

    def bias_rmsnorm(self, out, bias, w, eps):
        """Bias then RMSNorm over rows, per column: (z fp32, inv64 fp64 per
        column, y64 fp64).  out: N x B fp32; bias, w: N fp32 or None."""
        out = np.ascontiguousarray(out, dtype=np.float32)
        N, B = out.shape
        args = []
        for v in (bias, w):
            if v is None:
                args.append(None)
            else:
                v = np.ascontiguousarray(v, dtype=np.float32)
                if v.shape != (N,):
                    raise ValueError("bias / weight must hold N values")
                args.append(v)
        z = np.empty((N, B), np.float32)
        inv = np.empty(B, np.float64)
        y = np.empty((N, B), np.float64)
        rc = self._lib.gsa_oracle_bias_rmsnorm(
            _ptr(out, _f32p), None if args[0] is None else _ptr(args[0], _f32p),
            None if args[1] is None else _ptr(args[1], _f32p), float(eps), N, B,
            _ptr(z, _f32p), _ptr(inv, _f64p), _ptr(y, _f64p))
        if rc != 0:
            raise ValueError("oracle rejected the arguments")
        return z, inv, y

    def scale_f32(self, z, inv, w):
        """y = fl32(fl32(z * inv[b]) * w[n]) and its bf16 bits (RNE)."""
        z = np.ascontiguousarray(z, dtype=np.float32)
        N, B = z.shape
        inv = np.ascontiguousarray(inv, dtype=np.float32)
        if inv.shape != (B,):
            raise ValueError("inv must hold B values")
        wp = None
        if w is not None:
            w = np.ascontiguousarray(w, dtype=np.float32)
            wp = _ptr(w, _f32p)
        y = np.empty((N, B), np.float32)
        yb = np.empty((N, B), np.uint16)
        self._lib.gsa_oracle_scale_f32(_ptr(z, _f32p), _ptr(inv, _f32p), wp, N, B,
                                       _ptr(y, _f32p), _ptr(yb, _u16p))
        return y, yb

    def two_shot_chunk_rows(self, N, W):
        """Rows per rank's chunk in the two-shot variant (whole 16-row tiles)."""
        return int(self._lib.gsa_oracle_two_shot_chunk_rows(N, W))

    def two_shot(self, slots, gathered, rank):
        """(out, mine): out rows of the own chunk = fp32 rank-order fold of the
        slots, other rows = gathered; mine = the own chunk's published values
        (NaN elsewhere).  slots: W x N x B fp32; gathered: N x B fp32."""
        slots = np.ascontiguousarray(slots, dtype=np.float32)
        W, N, B = slots.shape
        gathered = np.ascontiguousarray(gathered, dtype=np.float32)
        if gathered.shape != (N, B):
            raise ValueError("gathered must be N x B")
        out = np.empty((N, B), np.float32)
        mine = np.full((N, B), np.nan, np.float32)
        self._lib.gsa_oracle_two_shot(_ptr(slots, _f32p), _ptr(gathered, _f32p), W, rank, N, B,
                                      _ptr(out, _f32p), _ptr(mine, _f32p))
        return out, mine

    def moe_combine(self, X, Wd, length, in_off, dst_off, W, rows_out):
        """Expert products placed by the combine all-to-all, at one rank's
        share: (y64, abs64, written) with y64 / abs64 float64 W x rows_out x H
        (NaN where no segment lands) and written uint8 W x rows_out.

        X: uint16 bf16 bits rows_in x F; Wd: uint16 ne x H x F; length and
        in_off: int ne x W; dst_off: int W x ne.  Raises ValueError on a
        segment out of range (-1) or two segments on one row (-2)."""
        X = np.ascontiguousarray(X, dtype=np.uint16)
        Wd = np.ascontiguousarray(Wd, dtype=np.uint16)
        ne, H, F = Wd.shape
        rows_in = X.shape[0]
        if X.shape[1] != F:
            raise ValueError("X and Wd disagree on F")
        length = np.ascontiguousarray(length, dtype=np.int32).reshape(ne, W)
        in_off = np.ascontiguousarray(in_off, dtype=np.int32).reshape(ne, W)
        dst_off = np.ascontiguousarray(dst_off, dtype=np.int32).reshape(W, ne)
        y = np.full((W, rows_out, H), np.nan)
        a = np.full((W, rows_out, H), np.nan)
        written = np.zeros((W, rows_out), np.uint8)
        rc = self._lib.gsa_oracle_moe_combine(
            _ptr(X, _u16p), _ptr(Wd, _u16p), _ptr(length, self._i32p), _ptr(in_off, self._i32p),
            _ptr(dst_off, self._i32p), W, ne, H, F, rows_in, rows_out, _ptr(y, _f64p),
            _ptr(a, _f64p), written.ctypes.data_as(ctypes.POINTER(ctypes.c_uint8)))
        if rc != 0:
            raise ValueError(f"oracle rejected the segments ({rc})")
        return y, a, written

    def fold_f32(self, slots):
        """fp32 one-shot sum of the given slots in rank order from +0.0f."""
        slots = np.ascontiguousarray(slots, dtype=np.float32)
        W = slots.shape[0]
        rest = slots.shape[1:]
        nb = int(np.prod(rest)) if rest else 1
        out = np.empty(rest, np.float32)
        self._lib.gsa_oracle_fold_f32(_ptr(slots, _f32p), W, nb, _ptr(out, _f32p))
        return out

    def fold_bf16(self, slots):
        """fp32 one-shot sum of bf16 slots (uint16 bits, W x ...), each
        widened exactly, in rank order from +0.0f."""
        slots = np.ascontiguousarray(slots, dtype=np.uint16)
        W = slots.shape[0]
        rest = slots.shape[1:]
        nb = int(np.prod(rest)) if rest else 1
        out = np.empty(rest, np.float32)
        self._lib.gsa_oracle_fold_bf16(_ptr(slots, _u16p), W, nb, _ptr(out, _f32p))
        return out

    def to_bf16(self, v):
        """bf16 bits (uint16) of float32 values, round to nearest, ties to even."""
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.empty(v.shape, np.uint16)
        self._lib.gsa_oracle_f32_to_bf16(_ptr(v, _f32p), int(v.size), _ptr(out, _u16p))
        return out


def bound(abs64):
    """Allowed |fp32 result - fp64 value| for each element."""
    return BOUND_REL * np.asarray(abs64, np.float64) + BOUND_ABS


def bound_bf16(abs64, y64):
    """Allowed |bf16 result - fp64 value| when an fp32 result within bound()
    is then rounded to bf16: a bf16 value carries 8 significant bits, so
    round-to-nearest moves v by at most half a unit in its last place, which
    is at most 2^-8 |v|; with |v| <= |y64| + bound this adds
    2^-8 (|y64| + bound) to bound()."""
    b = bound(abs64)
    return b + 2.0 ** -8 * (np.abs(np.asarray(y64, np.float64)) + b)


def flag_tiles(N):
    """Number of flag tiles for N output rows."""
    return (int(N) + FLAG_TILE_ROWS - 1) // FLAG_TILE_ROWS


def pad_after_reset(W, N, published_mask):
    """Logical W x T flag state right after a reset: published rows hold the
    all-ones word, every other row holds 0."""
    T = flag_tiles(N)
    flags = np.zeros((W, T), np.uint32)
    for p in range(W):
        if (published_mask >> p) & 1:
            flags[p, :] = FLAG_PUBLISHED
    return flags


def pad_after_calls(flags, rank, calls):
    """State after `calls` calls by `rank` that each completed: a call whose
    own flag read f publishes f + 1 (the call's epoch) on every tile of its
    own row; peer rows are only read."""
    flags = np.array(flags, np.uint32, copy=True)
    flags[rank, :] = flags[rank, :] + np.uint32(calls)
    return flags


def expected_timeouts(flags_before, rank):
    """Which (tile, peer) waits of one call cannot be satisfied, given the pad
    before the call.  Epoch e_t = own flag + 1; the wait on peer p for tile t
    needs flags[p][t] >= e_t.  Returns (timed_out_tiles, first) where first is
    the lexicographically smallest (tile, peer) pair, or None."""
    flags_before = np.asarray(flags_before, np.uint64)
    W, T = flags_before.shape
    epoch = flags_before[rank] + 1
    tiles = []
    first = None
    for t in range(T):
        missing = [p for p in range(W) if p != rank and flags_before[p, t] < epoch[t]]
        if missing:
            tiles.append(t)
            if first is None:
                first = (t, missing[0])
    return tiles, first


_default = None


def load(path=None):
    """Load the oracle library (building it first if it is not built)."""
    global _default
    if path is not None:
        return Oracle(path)
    if _default is None:
        if not os.path.exists(_build.LIBRARY) or (
                os.path.getmtime(_build.LIBRARY) < os.path.getmtime(_build.SOURCE)):
            _build.build()
        _default = Oracle(_build.LIBRARY)
    return _default
