"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an `oracle.Oracle` and raises AssertionError on a mismatch.
They are collected by test_oracle_pins.py (against the real oracle) and by
test_oracle_mutants.py (against copies with planted mistakes, each of which
must fail at least one pin).

What pins what:
  brute_force      GEMV, abs-sum and one-shot sum vs numpy fp64 matmul and
                   numpy sums on tiny shapes (textbook routine, other order)
  single_rank      W = 1: out equals the unsharded product
  shard_sum        sum over shards of y_r equals the full product
  identity         A = I gives y = x exactly
  one_hot          x = e_j gives y = A[:, j] exactly
  small_integers   integer-valued A, x: exact integer results (int64 matmul)
  rank_order_exact own term is y, slot[rank] is ignored, peers enter once
  bf16_decode      raw bits to value, incl. denormal and max finite
  golden           hand-worked example in tests/golden/ (values by hand)
  fold_*           fp32 fold: order, +0 start and fp32 rounding, by hand
  rms_golden       bias + RMSNorm hand-worked example in tests/golden/
  rms_*            RMSNorm closed forms and invariants: constant column,
                   unit RMS at eps = 0, scale invariance, bias cancelling,
                   independent columns
  scale_exact      fp32 evaluation of the normalised output against exact
                   rational arithmetic with IEEE round-to-nearest-even
  bf16_rne         fp32 -> bf16 rounding, hand-chosen bit patterns
  bf16_reduce_*    the all-reduce over bf16 slots with fp32 accumulation and
                   bf16 output: a hand-worked golden file (cases where bf16
                   accumulation, another order or another start would give
                   other bits), numpy float32 scalar adds in rank order, and
                   the rounding built from the definition (the nearer of the
                   two neighbouring bf16 values, ties to the even one)
  two_shot_*       chunk partition (hand values and its defining properties),
                   ownership of every row for every rank against numpy
                   float32 sums in rank order and plain copies
  moe_*            the MoE product + combine placement: numpy fp64 matmul of
                   every segment placed by slicing, identity weights (rows
                   move exactly), one-hot rows (pick a weight column), a
                   hand-worked golden file, rejection of overlapping and
                   out-of-range segments
"""
from fractions import Fraction
import json
import os

import numpy as np

import gsa_inputs as gi

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f64(bits):
    return gi.bf16_bits_to_f32(bits).astype(np.float64)


def _close(a, b, rel, scale, what):
    err = np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))
    lim = rel * np.asarray(scale, np.float64) + 1e-300
    bad = ~(err <= lim)
    assert not bad.any(), f"{what}: {int(bad.sum())} elements off, max err {err.max():.3e}"


def pin_brute_force(o):
    rng = np.random.default_rng(1234)
    for (N, Ks, B, W) in [(8, 8, 1, 1), (17, 24, 2, 2), (33, 40, 3, 3),
                          (64, 64, 16, 8), (40, 56, 2, 8), (9, 16, 3, 2)]:
        for rank in sorted({0, W - 1, W // 2}):
            A = gi.bf16_bits(rng.normal(0, 0.5, (N, Ks)).astype(np.float32))
            x = gi.bf16_bits(rng.normal(0, 1.0, (B, Ks)).astype(np.float32))
            slots = rng.normal(0, 1, (W, N, B)).astype(np.float32)
            slots[rank] = np.nan
            y, a, out = o.gemv_allreduce(A, x, slots, rank)
            Af, xf = _f64(A), _f64(x)
            ref = Af @ xf.T
            ref_abs = np.abs(Af) @ np.abs(xf).T
            _close(y, ref, 1e-13, ref_abs, "y vs numpy")
            _close(a, ref_abs, 1e-13, ref_abs, "abs vs numpy")
            peers = [slots[r].astype(np.float64) for r in range(W) if r != rank]
            ref_out = ref + (np.sum(peers, axis=0) if peers else 0.0)
            scale = ref_abs + sum(np.abs(p) for p in peers) if peers else ref_abs
            _close(out, ref_out, 1e-13, scale, "out vs numpy")


def pin_single_rank(o):
    rng = np.random.default_rng(7)
    N, K, B = 24, 48, 3
    A = gi.bf16_bits(rng.normal(0, 0.1, (N, K)).astype(np.float32))
    x = gi.bf16_bits(rng.normal(0, 1, (B, K)).astype(np.float32))
    slots = np.full((1, N, B), np.nan, np.float32)
    y, a, out = o.gemv_allreduce(A, x, slots, 0)
    assert np.array_equal(out, y), "W=1: out must equal y"
    ref = _f64(A) @ _f64(x).T
    _close(out, ref, 1e-13, np.abs(_f64(A)) @ np.abs(_f64(x)).T, "W=1 vs unsharded")


def pin_shard_sum(o):
    A, x = gi.make_full_inputs(32, 96, 2, sigma=0.3, seed=5)
    ref = _f64(A) @ _f64(x).T
    scale = np.abs(_f64(A)) @ np.abs(_f64(x)).T
    for W in (2, 3, 4, 8):
        total = np.zeros_like(ref)
        for r in range(W):
            Ar, xr = gi.shard(A, x, W, r)
            y, _ = o.gemv(Ar, xr)
            total += y
        _close(total, ref, 1e-13, scale, f"shard sum W={W}")


def pin_identity(o):
    Ks = 24
    one = gi.bf16_bits(np.array([1.0], np.float32))[0]
    A = np.zeros((Ks, Ks), np.uint16)
    A[np.arange(Ks), np.arange(Ks)] = one
    rng = np.random.default_rng(3)
    x = gi.bf16_bits(rng.normal(0, 1, (3, Ks)).astype(np.float32))
    y, _ = o.gemv(A, x)
    assert np.array_equal(y, _f64(x).T), "identity: y must equal x"


def pin_one_hot(o):
    rng = np.random.default_rng(4)
    N, Ks, B = 20, 32, 4
    A = gi.bf16_bits(rng.normal(0, 1, (N, Ks)).astype(np.float32))
    one = gi.bf16_bits(np.array([1.0], np.float32))[0]
    cols = [0, 5, 17, Ks - 1]
    x = np.zeros((B, Ks), np.uint16)
    for b, j in enumerate(cols):
        x[b, j] = one
    y, _ = o.gemv(A, x)
    for b, j in enumerate(cols):
        assert np.array_equal(y[:, b], _f64(A)[:, j]), f"one-hot column {j}"


def pin_small_integers(o):
    rng = np.random.default_rng(5)
    N, Ks, B = 13, 40, 3
    Ai = rng.integers(-4, 5, (N, Ks))
    xi = rng.integers(-4, 5, (B, Ks))
    A = gi.bf16_bits(Ai.astype(np.float32))
    x = gi.bf16_bits(xi.astype(np.float32))
    y, a = o.gemv(A, x)
    assert np.array_equal(y, (Ai @ xi.T).astype(np.float64)), "integer products"
    assert np.array_equal(a, (np.abs(Ai) @ np.abs(xi).T).astype(np.float64)), "integer abs"


def pin_rank_order_exact(o):
    # Integer-valued peers: every sum is exact, so only the choice of terms
    # matters: y for the own rank, each peer slot once, slot[rank] ignored.
    N, Ks, B, W = 4, 8, 2, 4
    Ai = np.arange(N * Ks).reshape(N, Ks) % 5 - 2
    xi = np.arange(B * Ks).reshape(B, Ks) % 3 - 1
    A = gi.bf16_bits(Ai.astype(np.float32))
    x = gi.bf16_bits(xi.astype(np.float32))
    yi = Ai @ xi.T
    for rank in range(W):
        slots = np.empty((W, N, B), np.float32)
        for r in range(W):
            slots[r] = 1000.0 * (r + 1) + np.arange(N * B).reshape(N, B)
        slots[rank] = np.nan
        _, _, out = o.gemv_allreduce(A, x, slots, rank)
        ref = yi.astype(np.float64)
        for r in range(W):
            if r != rank:
                ref = ref + slots[r].astype(np.float64)
        assert np.array_equal(out, ref), f"rank {rank}: wrong set of terms"


def pin_bf16_decode(o):
    cases = {0x3F80: 1.0, 0xC040: -3.0, 0x0080: 2.0 ** -126,
             0x0001: 2.0 ** -133, 0x7F7F: float(np.float32(3.3895313892515355e38)),
             0x8000: -0.0, 0x4049: 3.140625}
    bits = np.array(list(cases.keys()), np.uint16)[:, None]
    one = gi.bf16_bits(np.array([[1.0]], np.float32))
    y, a = o.gemv(bits, one)
    assert np.array_equal(y[:, 0], np.array(list(cases.values()))), f"decode {y[:, 0]}"


def pin_golden(o):
    with open(os.path.join(GOLDEN, "hand_worked_w2.json")) as f:
        g = json.load(f)
    A = gi.bf16_bits(np.array(g["A"], np.float32))
    x = gi.bf16_bits(np.array(g["x"], np.float32))
    slots = np.array(g["slots"], np.float32)
    y, a, out = o.gemv_allreduce(A, x, slots, g["rank"])
    assert np.array_equal(y, np.array(g["y"], np.float64)), "golden y"
    assert np.array_equal(a, np.array(g["abs"], np.float64)), "golden abs"
    assert np.array_equal(out, np.array(g["out"], np.float64)), "golden out"


def _fold_bits(o, cols):
    """Fold columns given as lists of float32 values (one per rank)."""
    W = len(cols[0])
    slots = np.array(cols, np.float32).T.reshape(W, len(cols)).copy()
    return o.fold_f32(slots)


def pin_fold_order(o):
    big = float(2 ** 24)
    # ((0 + 2^24) + 1) + 1 = 2^24 in fp32 (each +1 is a tie, kept even);
    # the reverse order would give 2^24 + 2.
    # ((0 + 1) + 2^24) - 2^24 = 0 (2^24 + 1 rounds to 2^24); reverse gives 1.
    out = _fold_bits(o, [[big, 1.0, 1.0], [1.0, big, -big]])
    assert out[0] == np.float32(big) and out[1] == np.float32(0.0), f"fold order {out}"


def pin_fold_zero_start(o):
    # The sum starts from +0.0: (+0) + (-0) = +0 in round-to-nearest.
    out = _fold_bits(o, [[-0.0], [-0.0]])
    assert not np.signbit(out).any(), "fold must start from +0.0"
    out2 = _fold_bits(o, [[-0.0, -0.0, -0.0]])
    assert not np.signbit(out2[0]), "fold must start from +0.0 (W=3)"


def pin_fold_fp32(o):
    # 1 + 2^-24 is a tie in fp32 and rounds to 1; fp64 would keep it.
    # 1 + 3*2^-24 rounds up to 1 + 2^-22 (nearest).
    out = _fold_bits(o, [[1.0, 2.0 ** -24], [1.0, 3 * 2.0 ** -24]])
    assert out[0] == np.float32(1.0), f"fp32 tie: {out[0]!r}"
    assert out[1] == np.float32(1.0 + 2.0 ** -22), f"fp32 rounding: {out[1]!r}"


def pin_fold_matches_sequence(o):
    # Random case, checked element-wise against numpy float32 scalar adds in
    # rank order (numpy's float32 add is IEEE round-to-nearest).
    rng = np.random.default_rng(11)
    W, NB = 8, 257
    slots = (rng.normal(0, 1, (W, NB)) * rng.choice([1e-3, 1, 1e3], (W, NB))).astype(np.float32)
    out = o.fold_f32(slots)
    for i in range(NB):
        acc = np.float32(0.0)
        for r in range(W):
            acc = np.float32(acc + slots[r, i])
        assert out[i].view(np.uint32) == acc.view(np.uint32), f"fold element {i}"


def pin_rms_golden(o):
    with open(os.path.join(GOLDEN, "rmsnorm_hand.json")) as f:
        g = json.load(f)
    z, inv, y = o.bias_rmsnorm(np.array(g["out"], np.float32), np.array(g["bias"], np.float32),
                               np.array(g["weight"], np.float32), g["eps"])
    assert np.array_equal(z, np.array(g["z"], np.float32)), f"golden z {z}"
    _close(inv, g["inv"], 1e-15, np.abs(g["inv"]), "golden inv_rms")
    _close(y, g["y"], 1e-15, np.abs(np.array(g["y"])) + 1e-300, "golden y")


def pin_rms_constant_column(o):
    # A column holding one value c everywhere: inv = 1 / sqrt(c^2 + eps).
    N, eps = 37, 0.25
    cs = np.array([3.0, -0.5, 1024.0], np.float32)
    out = np.tile(cs, (N, 1))
    z, inv, y = o.bias_rmsnorm(out, None, None, eps)
    want = 1.0 / np.sqrt(cs.astype(np.float64) ** 2 + eps)
    _close(inv, want, 1e-14, want, "constant-column inv_rms")
    _close(y, np.tile(cs * want, (N, 1)), 1e-14, np.abs(np.tile(cs * want, (N, 1))),
           "constant-column y")


def pin_rms_unit_rms(o):
    # eps = 0, no weight: every normalised column has mean square 1.
    rng = np.random.default_rng(5)
    out = rng.normal(0, 3, (50, 4)).astype(np.float32)
    _, _, y = o.bias_rmsnorm(out, None, None, 0.0)
    ms = (y ** 2).mean(axis=0)
    assert np.all(np.abs(ms - 1.0) < 1e-12), f"unit RMS: {ms}"


def pin_rms_scale_invariant(o):
    # eps = 0: scaling a column by 4 (exact in fp32) leaves y unchanged, and
    # scales inv by 1/4.
    rng = np.random.default_rng(6)
    out = rng.normal(0, 1, (33, 3)).astype(np.float32)
    w = rng.normal(1, 0.1, 33).astype(np.float32)
    _, inv1, y1 = o.bias_rmsnorm(out, None, w, 0.0)
    _, inv4, y4 = o.bias_rmsnorm(out * np.float32(4), None, w, 0.0)
    _close(y4, y1, 1e-13, np.abs(y1) + 1e-30, "scale invariance of y")
    _close(inv4 * 4, inv1, 1e-14, inv1, "inv scales by 1/4")


def pin_rms_bias_cancels(o):
    # bias = -out on every row: z = 0, inv = 1/sqrt(eps), y = 0; and a bias
    # that shifts a constant column by a known amount.
    rng = np.random.default_rng(7)
    out = rng.normal(0, 1, (20, 1)).astype(np.float32)
    z, inv, y = o.bias_rmsnorm(out, -out[:, 0], None, 4.0)
    assert np.all(z == 0) and np.all(y == 0), "bias = -out gives zeros"
    assert inv[0] == 0.5, f"inv = 1/sqrt(eps) = 0.5, got {inv[0]}"
    z2, inv2, _ = o.bias_rmsnorm(np.full((8, 1), 1.0, np.float32),
                                 np.full(8, 2.0, np.float32), None, 0.0)
    assert np.all(z2 == 3.0) and abs(inv2[0] - 1.0 / 3.0) < 1e-16, "bias shifts z"


def pin_rms_columns_independent(o):
    # Each token column is normalised on its own: permuting columns permutes
    # the results, and columns do not leak into each other.
    rng = np.random.default_rng(8)
    out = rng.normal(0, 1, (24, 3)).astype(np.float32)
    out[:, 1] *= 100.0
    w = rng.normal(1, 0.2, 24).astype(np.float32)
    _, inv, y = o.bias_rmsnorm(out, None, w, 1e-3)
    perm = [2, 0, 1]
    _, invp, yp = o.bias_rmsnorm(np.ascontiguousarray(out[:, perm]), None, w, 1e-3)
    assert np.array_equal(invp, inv[perm]) and np.array_equal(yp, y[:, perm]), "column permutation"
    for b in range(3):
        _, i1, y1 = o.bias_rmsnorm(np.ascontiguousarray(out[:, b:b + 1]), None, w, 1e-3)
        assert i1[0] == inv[b] and np.array_equal(y1[:, 0], y[:, b]), f"column {b} alone"


def _rne_f32(q):
    """The fp32 value nearest to the exact rational q (ties to even), for q in
    the normal range: the IEEE rule restated on exact integers."""
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    q = abs(q)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    m = q / Fraction(2) ** (e - 23)          # in [2^23, 2^24)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(Fraction(fl) * Fraction(2) ** (e - 23))


def pin_scale_exact(o):
    # y = fl32(fl32(z * inv) * w): each product correctly rounded, in this
    # order, checked with exact rational arithmetic.  Random values near 1
    # make both roundings matter (and the other order differ on many).
    rng = np.random.default_rng(9)
    N, B = 64, 3
    z = rng.uniform(0.5, 2.0, (N, B)).astype(np.float32)
    inv = rng.uniform(0.5, 2.0, B).astype(np.float32)
    w = rng.uniform(0.5, 2.0, N).astype(np.float32)
    y, _ = o.scale_f32(z, inv, w)
    for n in range(N):
        for b in range(B):
            t = _rne_f32(Fraction(float(z[n, b])) * Fraction(float(inv[b])))
            want = _rne_f32(Fraction(t) * Fraction(float(w[n])))
            assert float(y[n, b]) == want, f"scale ({n},{b}): {float(y[n, b])!r} vs {want!r}"
    y0, _ = o.scale_f32(z, inv, None)
    for n in range(N):
        for b in range(B):
            want = _rne_f32(Fraction(float(z[n, b])) * Fraction(float(inv[b])))
            assert float(y0[n, b]) == want, f"scale without weight ({n},{b})"


def pin_bf16_rne(o):
    # fp32 bit pattern -> expected bf16 bits, chosen by hand.
    cases = [
        (0x3F800000, 0x3F80),  # 1.0
        (0x3F808000, 0x3F80),  # 1 + 2^-8: halfway, ties to even (down)
        (0x3F818000, 0x3F82),  # 1 + 3*2^-8: halfway, ties to even (up)
        (0x3F808001, 0x3F81),  # just above halfway: up
        (0x3F807FFF, 0x3F80),  # just below halfway: down
        (0xC0200000, 0xC020),  # -2.5, exact
        (0x7F7FFFFF, 0x7F80),  # largest finite fp32 rounds up to +inf
        (0x7F800000, 0x7F80),  # +inf
        (0x80000000, 0x8000),  # -0.0
        (0x00000001, 0x0000),  # smallest denormal rounds to +0
        (0x00010000, 0x0001),  # a bf16 denormal, exact
    ]
    bits = np.array([c[0] for c in cases], np.uint32)
    z = bits.view(np.float32).reshape(-1, 1)
    _, yb = o.scale_f32(z, np.ones(1, np.float32), None)
    got = [int(v) for v in yb[:, 0]]
    assert got == [c[1] for c in cases], f"bf16 rounding {[hex(v) for v in got]}"
    # A quiet NaN with an all-ones payload: adding the rounding increment
    # would carry into the sign and exponent; it must stay a NaN.
    nan = np.array([[np.uint32(0x7FFFFFFF).view(np.float32)]])
    _, ybn = o.scale_f32(nan, np.ones(1, np.float32), None)
    v = int(ybn[0, 0])
    assert (v & 0x7F80) == 0x7F80 and (v & 0x007F) != 0 and (v & 0x0040), \
        f"NaN stays a quiet NaN, got {hex(v)}"


def pin_bf16_reduce_golden(o):
    with open(os.path.join(GOLDEN, "bf16_allreduce_hand.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        bits = np.array([int(b, 16) for b in c["bits"]], np.uint16).reshape(-1, 1)
        fold = o.fold_bf16(bits)
        want = np.float32(c["fold_f32"])
        assert fold[0].view(np.uint32) == want.view(np.uint32), (
            f"bf16 slots {c['slots']}: fp32 fold {fold[0]!r}, want {want!r}")
        got = int(o.to_bf16(fold)[0])
        assert got == int(c["out_bits"], 16), (
            f"bf16 slots {c['slots']}: out bits {hex(got)}, want {c['out_bits']}")


def pin_bf16_reduce_sequence(o):
    # Random bf16 slots: widen each exactly (bits << 16) and add them in rank
    # order with numpy float32 scalar adds (IEEE round-to-nearest).
    rng = np.random.default_rng(12)
    W, NB = 8, 301
    vals = (rng.normal(0, 1, (W, NB)) * rng.choice([1e-3, 1, 1e3], (W, NB))).astype(np.float32)
    bits = gi.bf16_bits(vals)
    out = o.fold_bf16(bits)
    wide = (bits.astype(np.uint32) << 16).view(np.float32)
    for i in range(NB):
        acc = np.float32(0.0)
        for r in range(W):
            acc = np.float32(acc + wide[r, i])
        assert out[i].view(np.uint32) == acc.view(np.uint32), f"bf16 fold element {i}"


def _bf16_nearest_by_definition(v):
    """bf16 bits of the bf16 value nearest to the finite float32 v (ties: the
    one whose last stored bit is 0), found by comparing the distances to the
    two neighbours in exact arithmetic -- not by the rounding bit trick."""
    u = int(np.float32(v).view(np.uint32))
    lo = u >> 16                           # toward zero: the upper half of the word
    hi = lo + 1                            # the next bf16 value away from zero
    def val(b):
        return Fraction(float(np.uint32(b << 16).view(np.float32)))
    x = Fraction(float(v))
    d_lo, d_hi = abs(x - val(lo)), abs(val(hi) - x)
    if d_lo < d_hi:
        return lo
    if d_hi < d_lo:
        return hi
    return lo if lo % 2 == 0 else hi


def pin_bf16_reduce_rounding(o):
    rng = np.random.default_rng(13)
    v = (rng.normal(0, 1, 400) * rng.choice([1e-30, 1e-3, 1, 1e5, 1e30], 400)).astype(np.float32)
    # exact ties and their neighbours: upper halves with the low 16 bits
    # 0x8000 (halfway) and 0x7FFF / 0x8001
    base = rng.integers(0x0080, 0x7F00, 60).astype(np.uint32) << 16
    sign = rng.integers(0, 2, 60).astype(np.uint32) << 31
    for low in (0x8000, 0x7FFF, 0x8001):
        v = np.concatenate([v, ((base | sign) + low).view(np.float32)])
    got = o.to_bf16(v)
    for i, f in enumerate(v):
        want = _bf16_nearest_by_definition(f)
        assert int(got[i]) == want, f"bf16 of {f!r}: {hex(int(got[i]))}, want {hex(want)}"


def pin_two_shot_chunks(o):
    # Hand values: ceil(N / W) rounded up to whole 16-row tiles.
    for N, W, want in [(4096, 8, 512), (17, 8, 16), (1000, 3, 336), (33, 2, 32), (1, 1, 16),
                       (16384, 8, 2048), (8192, 4, 2048), (4097, 8, 528)]:
        got = o.two_shot_chunk_rows(N, W)
        assert got == want, f"chunk rows N={N} W={W}: {got} != {want}"
    # Defining properties on a sweep: a multiple of 16, every row owned, and
    # the smallest such size.
    for N in (1, 15, 16, 17, 100, 1023, 4096, 5000):
        for W in range(1, 9):
            cr = o.two_shot_chunk_rows(N, W)
            per = -(-N // W)
            assert cr % 16 == 0 and cr >= per and cr - 16 < per and W * cr >= N, (N, W, cr)


def pin_two_shot_rows(o):
    # For every rank: rows of its chunk hold the float32 rank-order sum of
    # the slots (numpy scalar adds), every other row a copy of gathered.
    rng = np.random.default_rng(13)
    W, N, B = 3, 70, 2
    slots = rng.normal(0, 1, (W, N, B)).astype(np.float32)
    gathered = rng.normal(0, 1, (N, B)).astype(np.float32)
    cr = -(-(-(-N // W)) // 16) * 16
    for rank in range(W):
        out, mine = o.two_shot(slots, gathered, rank)
        for n in range(N):
            own = rank * cr <= n < (rank + 1) * cr
            for b in range(B):
                if own:
                    acc = np.float32(0.0)
                    for r in range(W):
                        acc = np.float32(acc + slots[r, n, b])
                    assert out[n, b].view(np.uint32) == acc.view(np.uint32), (rank, n, b)
                    assert mine[n, b].view(np.uint32) == acc.view(np.uint32), (rank, n, b)
                else:
                    assert out[n, b].view(np.uint32) == gathered[n, b].view(np.uint32), (rank, n, b)
                    assert np.isnan(mine[n, b]), (rank, n, b)


def _moe_call(o, d):
    return o.moe_combine(d["X"], d["Wd"], d["length"], d["in_off"], d["dst_off"], d["W"],
                         d["rows_out"])


def _tiny_moe(seed, W=3, ne=2, H=5, F=7, max_len=3, gap=1):
    """Random tiny MoE call: random segment lengths (zeros included), gaps
    between segments in X, destinations packed in rank s's buffer in global
    expert order with a random start."""
    rng = np.random.default_rng(seed)
    length = rng.integers(0, max_len + 1, size=(ne, W)).astype(np.int32)
    in_off = np.zeros((ne, W), np.int32)
    row = 0
    for e in range(ne):
        for s in range(W):
            in_off[e, s] = row
            row += int(length[e, s]) + gap
    dst_off = np.zeros((W, ne), np.int32)
    rows_out = 0
    for s in range(W):
        at = int(rng.integers(0, 3))
        for e in range(ne):
            dst_off[s, e] = at
            at += int(length[e, s])
        rows_out = max(rows_out, at + 1)
    X = gi.bf16_bits(rng.normal(0, 1, size=(max(row, 1), F)).astype(np.float32))
    Wd = gi.bf16_bits(rng.normal(0, 1, size=(ne, H, F)).astype(np.float32))
    return dict(X=X, Wd=Wd, length=length, in_off=in_off, dst_off=dst_off, W=W, ne=ne, H=H, F=F,
                rows_out=rows_out)


def pin_moe_numpy(o):
    # Against numpy float64 matmul of each segment, placed by plain slicing.
    for seed in range(4):
        d = _tiny_moe(seed)
        y, a, written = _moe_call(o, d)
        want = np.full_like(y, np.nan)
        wabs = np.full_like(y, np.nan)
        X = gi.bf16_bits_to_f32(d["X"]).astype(np.float64)
        Wd = gi.bf16_bits_to_f32(d["Wd"]).astype(np.float64)
        for e in range(d["ne"]):
            for s in range(d["W"]):
                n, src, dst = d["length"][e, s], d["in_off"][e, s], d["dst_off"][s, e]
                seg = X[src:src + n]
                want[s, dst:dst + n] = seg @ Wd[e].T
                wabs[s, dst:dst + n] = np.abs(seg) @ np.abs(Wd[e]).T
        assert np.array_equal(np.isnan(y), np.isnan(want)), "rows placed differently"
        m = ~np.isnan(want)
        assert np.allclose(y[m], want[m], rtol=1e-12, atol=1e-12), "moe values"
        assert np.allclose(a[m], wabs[m], rtol=1e-12, atol=1e-12), "moe abs sums"
        assert int(written.sum()) == int(d["length"].sum()), "rows written"


def pin_moe_identity(o):
    # Identity weights (H = F): every destination row is its source X row,
    # exactly; rows are told apart by their values.
    d = _tiny_moe(11, W=4, ne=3, H=6, F=6)
    eye = gi.bf16_bits(np.eye(6, dtype=np.float32))
    d["Wd"] = np.stack([eye] * d["ne"])
    y, a, written = _moe_call(o, d)
    X = gi.bf16_bits_to_f32(d["X"]).astype(np.float64)
    for s in range(d["W"]):
        for e in range(d["ne"]):
            for i in range(int(d["length"][e, s])):
                src = int(d["in_off"][e, s]) + i
                dst = int(d["dst_off"][s, e]) + i
                assert np.array_equal(y[s, dst], X[src]), (s, e, i)


def pin_moe_one_hot(o):
    # A one-hot source row picks one input column of the expert's weight.
    d = _tiny_moe(12, W=2, ne=2, H=4, F=5, max_len=2, gap=0)
    F = d["F"]
    rows = d["X"].shape[0]
    hot = [(r * 3 + 1) % F for r in range(rows)]
    X = np.zeros((rows, F), np.float32)
    X[np.arange(rows), hot] = 1.0
    d["X"] = gi.bf16_bits(X)
    y, a, written = _moe_call(o, d)
    Wd = gi.bf16_bits_to_f32(d["Wd"]).astype(np.float64)
    for s in range(d["W"]):
        for e in range(d["ne"]):
            for i in range(int(d["length"][e, s])):
                src = int(d["in_off"][e, s]) + i
                dst = int(d["dst_off"][s, e]) + i
                assert np.array_equal(y[s, dst], Wd[e][:, hot[src]]), (s, e, i)


def pin_moe_golden(o):
    with open(os.path.join(GOLDEN, "moe_hand.json")) as f:
        g = json.load(f)
    X = gi.bf16_bits(np.array(g["X"], np.float32))
    Wd = gi.bf16_bits(np.array(g["Wd"], np.float32))
    y, a, written = o.moe_combine(X, Wd, np.array(g["length"]), np.array(g["in_off"]),
                                  np.array(g["dst_off"]), g["W"], g["rows_out"])
    for key, row in g["expect"].items():
        s, r = map(int, key.split(","))
        assert np.array_equal(y[s, r], np.array(row)), f"golden moe {key}"
        assert np.array_equal(a[s, r], np.array(g["expect_abs"][key])), f"golden moe abs {key}"
    assert int(written.sum()) == len(g["expect"]), "golden moe rows written"


def pin_moe_rejects(o):
    # Two segments on one destination row, and a segment past the buffer.
    d = _tiny_moe(13, W=2, ne=2, H=3, F=4, max_len=2, gap=0)
    d["length"][:] = 1
    d["in_off"] = np.arange(4, dtype=np.int32).reshape(2, 2)
    d["X"] = d["X"][:1].repeat(4, axis=0)
    d["dst_off"] = np.array([[0, 0], [0, 1]], np.int32)  # rank 0: both experts on row 0
    d["rows_out"] = 2
    try:
        _moe_call(o, d)
        raise AssertionError("overlap not rejected")
    except ValueError as e:
        assert "(-2)" in str(e), e
    d["dst_off"] = np.array([[0, 1], [0, 2]], np.int32)  # rank 1, expert 1: row 2 of 2
    try:
        _moe_call(o, d)
        raise AssertionError("out-of-range segment not rejected")
    except ValueError as e:
        assert "(-1)" in str(e), e


PINS = [pin_brute_force, pin_single_rank, pin_shard_sum, pin_identity, pin_one_hot,
        pin_small_integers, pin_rank_order_exact, pin_bf16_decode, pin_golden,
        pin_fold_order, pin_fold_zero_start, pin_fold_fp32, pin_fold_matches_sequence,
        pin_rms_golden, pin_rms_constant_column, pin_rms_unit_rms, pin_rms_scale_invariant,
        pin_rms_bias_cancels, pin_rms_columns_independent, pin_scale_exact, pin_bf16_rne,
        pin_bf16_reduce_golden, pin_bf16_reduce_sequence, pin_bf16_reduce_rounding,
        pin_two_shot_chunks, pin_two_shot_rows, pin_moe_numpy, pin_moe_identity,
        pin_moe_one_hot, pin_moe_golden, pin_moe_rejects]


def failing_pins(o):
    """Names of the pins that fail (or crash) for oracle build `o`."""
    bad = []
    for pin in PINS:
        try:
            pin(o)
        except Exception as e:  # noqa: BLE001 - any failure counts
            bad.append((pin.__name__, repr(e)[:200]))
    return bad
