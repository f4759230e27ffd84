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
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


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
