"""Seeded synthetic inputs for one rank's fused GEMV + one-shot AllReduce.

This module holds only random-number generation, bf16 rounding of the drawn
values and the workload table.  It contains none of the method's arithmetic;
the oracle and the HIP path both take its arrays as inputs.

Workloads (decode shapes of tensor-parallel Llama-class layers, W ranks,
A_r = this rank's N x K/W bf16 shard of the weight, x = this rank's B x K/W
bf16 slice of the activation, W-1 peer slots of N x B fp32 partial sums):

  c1   W=2 N=1024 K=1024  B=1   A~N(0,0.02)   small smoke case
  c2   W=8 N=4096 K=4096  B=1   A~N(0,0.02)   Llama-3-8B o_proj decode
  c3b* W=8 N=4096 K=14336 B=1/4/8 A~N(0,0.02) Llama-3-8B MLP down_proj
  c4   W=8 N=8192 K=28672 B=4   A~N(0,0.015)  70B-class MLP down_proj
  c5   W=4 N=8192 K=8192  B=16  A~N(0,0.02)   skinny GEMM (matrix-core path)

x ~ N(0, 1); peer slots ~ N(0, 1) fp32; for the two-shot variant the other
ranks' reduced chunks ~ N(0, 1) fp32.  No weights or datasets are used:
these draws stand in for the layer shapes named above.
"""
import numpy as np

CONFIGS = {
    "c1": dict(cfg_id=0, W=2, N=1024, K=1024, B=1, sigma=0.02,
               name="W=2 simulated ranks, 1024x512 shard, B=1"),
    "c2": dict(cfg_id=1, W=8, N=4096, K=4096, B=1, sigma=0.02,
               name="Llama-3-8B o_proj decode, W=8 N=4096 K=4096 B=1"),
    "c3b1": dict(cfg_id=2, W=8, N=4096, K=14336, B=1, sigma=0.02,
                 name="Llama-3-8B MLP down_proj, W=8 N=4096 K=14336 B=1"),
    "c3b4": dict(cfg_id=2, W=8, N=4096, K=14336, B=4, sigma=0.02,
                 name="Llama-3-8B MLP down_proj, W=8 N=4096 K=14336 B=4"),
    "c3b8": dict(cfg_id=2, W=8, N=4096, K=14336, B=8, sigma=0.02,
                 name="Llama-3-8B MLP down_proj, W=8 N=4096 K=14336 B=8"),
    "c4": dict(cfg_id=3, W=8, N=8192, K=28672, B=4, sigma=0.015,
               name="70B-class MLP down_proj, W=8 N=8192 K=28672 B=4"),
    "c5": dict(cfg_id=4, W=4, N=8192, K=8192, B=16, sigma=0.02,
               name="skinny GEMM, W=4 N=8192 K=8192 B=16"),
}

# Quiet-NaN bit pattern written into buffers the call must overwrite, so a
# missed write shows up as NaN.
SENTINEL_BITS = 0x7FC00000


def bf16_bits(values):
    """Round float values to bf16 (round to nearest, ties to even) and return
    the 16 raw bits as uint16.  Values must be finite."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    if not np.all(np.isfinite(f)):
        raise ValueError("bf16_bits needs finite values")
    u = f.view(np.uint32)
    # finite words are at most 0xFF7FFFFF, so the sum stays below 2^32
    r = (u >> 16) & 1
    r += 0x7FFF
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits):
    """Widen bf16 bits to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def sentinel(shape):
    """float32 array filled with the quiet-NaN sentinel."""
    return np.full(shape, SENTINEL_BITS, np.uint32).view(np.float32)


def _streams(seed, cfg_id):
    ss = np.random.SeedSequence([int(seed), int(cfg_id)])
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]


def make_shard_inputs(W, N, Ks, B, sigma=0.02, seed=0, cfg_id=0, rank=0):
    """One rank's inputs for an arbitrary shape.

    Returns dict with A (uint16 N x Ks), x (uint16 B x Ks) and slots
    (float32 W x N x B: peer rows ~N(0,1), row `rank` = NaN sentinel).
    """
    ga, gx, gp = _streams(seed, cfg_id)
    A = bf16_bits(ga.normal(0.0, sigma, size=(N, Ks)).astype(np.float32))
    x = bf16_bits(gx.normal(0.0, 1.0, size=(B, Ks)).astype(np.float32))
    slots = gp.normal(0.0, 1.0, size=(W, N, B)).astype(np.float32)
    slots[rank] = sentinel((N, B))
    return dict(A=A, x=x, slots=slots, W=W, N=N, Ks=Ks, K=Ks * W, B=B, rank=rank)


def make_inputs(cfg, seed=0, rank=0):
    """Inputs of a named workload (see CONFIGS) for `rank`."""
    c = CONFIGS[cfg] if isinstance(cfg, str) else cfg
    W, N, K, B = c["W"], c["N"], c["K"], c["B"]
    if K % W:
        raise ValueError("K must split evenly over W ranks")
    d = make_shard_inputs(W, N, K // W, B, c["sigma"], seed, c["cfg_id"] * 16 + B, rank)
    d["sigma"] = c["sigma"]
    return d


def make_gathered(N, B, seed=0, cfg_id=0):
    """Stand-in for the reduced chunks other ranks publish in the two-shot
    variant: float32 N x B ~ N(0, 1).  (The rows of the calling rank's own
    chunk are overwritten by the call; tests fill them with the sentinel.)"""
    ss = np.random.SeedSequence([int(seed), int(cfg_id), 2])
    g = np.random.Generator(np.random.PCG64(ss))
    return g.normal(0.0, 1.0, size=(N, B)).astype(np.float32)


def make_full_inputs(N, K, B, sigma=0.02, seed=0, cfg_id=99):
    """Unsharded A (N x K) and x (B x K) as bf16 bits, for shard-sum checks."""
    ga, gx, _ = _streams(seed, cfg_id)
    A = bf16_bits(ga.normal(0.0, sigma, size=(N, K)).astype(np.float32))
    x = bf16_bits(gx.normal(0.0, 1.0, size=(B, K)).astype(np.float32))
    return A, x


def shard(A, x, W, r):
    """Rank r's input-dimension slices of an unsharded A and x."""
    K = A.shape[1]
    Ks = K // W
    return (np.ascontiguousarray(A[:, r * Ks:(r + 1) * Ks]),
            np.ascontiguousarray(x[:, r * Ks:(r + 1) * Ks]))


# ---------------------------------------------------------------------------
# Mixture-of-experts workloads: the expert down-projection fused with the
# combine all-to-all, at one rank's share.  W ranks hold ne experts each
# (global expert g = rank * ne + e); every rank has T tokens, each routed to
# top_k distinct experts drawn uniformly; every assignment is kept (the pages
# name no capacity limit).  Weights ~ N(0, sigma), dispatched token rows
# ~ N(0, 1), bf16.
#
#   m0  W=4 ne=4  H=256  F=128  top-2 of 16,  T=8   small case
#   m1  W=8 ne=16 H=2048 F=768  top-8 of 128, T=16  Qwen3-30B-A3B-like down_proj
#   m2  W=8 ne=32 H=7168 F=2048 top-8 of 256, T=16  DeepSeek-V3-like down_proj
#   m3  W=8 ne=16 H=2048 F=768  top-8 of 128, T=64  the Qwen3-like shape with 64
#                                                   tokens per rank (about 32 per
#                                                   expert)
MOE_CONFIGS = {
    "m0": dict(cfg_id=20, W=4, ne=4, H=256, F=128, top_k=2, T=8, sigma=0.05,
               name="small MoE, W=4 ne=4 H=256 F=128 top-2 of 16, 8 tokens per rank"),
    "m1": dict(cfg_id=21, W=8, ne=16, H=2048, F=768, top_k=8, T=16, sigma=0.02,
               name="Qwen3-30B-A3B-like MoE down_proj, W=8 ne=16 H=2048 F=768 top-8 of 128, "
                    "16 tokens per rank"),
    "m2": dict(cfg_id=22, W=8, ne=32, H=7168, F=2048, top_k=8, T=16, sigma=0.02,
               name="DeepSeek-V3-like MoE down_proj, W=8 ne=32 H=7168 F=2048 top-8 of 256, "
                    "16 tokens per rank"),
    "m3": dict(cfg_id=23, W=8, ne=16, H=2048, F=768, top_k=8, T=64, sigma=0.02,
               name="Qwen3-30B-A3B-like MoE down_proj, W=8 ne=16 H=2048 F=768 top-8 of 128, "
                    "64 tokens per rank"),
}


def moe_routing(W, ne, T, top_k, seed=0, cfg_id=0):
    """Seeded routing of every rank's T tokens to top_k distinct experts each:
    counts[s][g] = tokens of rank s routed to global expert g (int64,
    W x W*ne); every row sums to T * top_k."""
    E = W * ne
    ss = np.random.SeedSequence([int(seed), int(cfg_id), 7])
    g = np.random.Generator(np.random.PCG64(ss))
    counts = np.zeros((W, E), np.int64)
    for s in range(W):
        for _ in range(T):
            experts = np.argsort(g.random(E))[:top_k]
            counts[s, experts] += 1
    return counts


def make_moe_inputs(cfg, seed=0, rank=0, gap=0):
    """One rank's inputs for a MoE workload (see MOE_CONFIGS): the seeded
    routing of moe_routing, then make_moe_from_counts."""
    c = MOE_CONFIGS[cfg] if isinstance(cfg, str) else cfg
    counts = moe_routing(c["W"], c["ne"], c["T"], c["top_k"], seed, c["cfg_id"])
    return make_moe_from_counts(counts, c["ne"], c["H"], c["F"], c["sigma"], seed, c["cfg_id"],
                                rank, gap, rows_out=c["T"] * c["top_k"])


def make_moe_from_counts(counts, ne, H, F, sigma=0.02, seed=0, cfg_id=0, rank=0, gap=0,
                         rows_out=None):
    """One rank's inputs given counts[s][g] (tokens of rank s accepted by
    global expert g, W x W*ne).

    Returns a dict with
      X        uint16 rows_in x F   dispatched token rows (bf16 bits), laid
                                    out expert-major then source-rank-major,
                                    `gap` unused rows after every segment
      Wd       uint16 ne x H x F    the rank's expert weights (bf16 bits)
      length   int32 ne x W         rows of source rank s for local expert e
      in_off   int32 ne x W         first row of that segment in X
      dst_off  int32 W x ne         first row of that segment in rank s's
                                    combine buffer (rank s's rows ordered by
                                    global expert)
      bufs     float32 W x rows_out x H: every rank's combine buffer before
               the call: rows of other ranks' experts ~ N(0, 1) (as if their
               owners had pushed them), this rank's rows NaN sentinel
    """
    counts = np.asarray(counts, np.int64)
    W = counts.shape[0]
    length = np.zeros((ne, W), np.int32)
    in_off = np.zeros((ne, W), np.int32)
    dst_off = np.zeros((W, ne), np.int32)
    row = 0
    for e in range(ne):
        for s in range(W):
            length[e, s] = counts[s, rank * ne + e]
            in_off[e, s] = row
            row += int(length[e, s]) + gap
    rows_in = max(row, 1)
    if rows_out is None:
        rows_out = max(1, int(counts.sum(axis=1).max()))
    for s in range(W):
        before = np.concatenate([[0], np.cumsum(counts[s])])
        for e in range(ne):
            dst_off[s, e] = before[rank * ne + e]
    ss = np.random.SeedSequence([int(seed), int(cfg_id), int(rank), 8])
    gw, gx, gb = [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(3)]
    w32 = gw.standard_normal(size=(ne, H, F), dtype=np.float32)
    w32 *= np.float32(sigma)
    Wd = bf16_bits(w32)
    del w32
    X = bf16_bits(gx.standard_normal(size=(rows_in, F), dtype=np.float32))
    bufs = gb.normal(0.0, 1.0, size=(W, rows_out, H)).astype(np.float32)
    for s in range(W):
        for e in range(ne):
            o, n = int(dst_off[s, e]), int(length[e, s])
            bufs[s, o:o + n] = sentinel((n, H))
    return dict(X=X, Wd=Wd, length=length, in_off=in_off, dst_off=dst_off, bufs=bufs, W=W,
                ne=ne, H=H, F=F, rows_in=rows_in, rows_out=rows_out, rank=rank, counts=counts)
