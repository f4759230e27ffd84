"""Benchmark: µs per gemv_allreduce call and achieved HBM GB/s on one MI355X.

One step = one fused call (GEMV of this rank's shard, publish, flag release,
one-shot reduce) on one batch of resident inputs.  The default workload is
the 70B-class MLP down_proj (W=8 N=8192 K=28672 B=4), the largest decode
shape of the workload table.

Inputs rotate over R independent sets whose total exceeds 1 GiB, so that a
call reads its set from HBM and not from the 256 MB Infinity Cache.  Order of
work (rank 0, N = 1):
  1. exactly --warmup untimed calls, on sets 0, 1, ... (mod R);
  2. a HIP graph is captured holding the K = --steps timed calls, which
     continue the rotation (call j on set (warmup + j) mod R);
  3. a 1 GiB read pass over a separate buffer evicts every set
     from the caches, and a bounded spin kernel keeps the GPU busy while the
     host queues the replay;
  4. the timed region: one graph replay between two HIP events recorded on
     the stream the kernels run on, between two device syncs.  The mean
     launch duration is the µs/call value and the denominator of the
     roofline figure.
So every timed call reads a set that has been untouched for at least 1 GiB
of other traffic, whatever K is.  Reported beside it, all measured after the
timed region: a second cold replay of the same graph (steps 3-4 again), an
eager pass of host-issued launches, a warm pass over one resident set
(Infinity-Cache resident, not HBM), and the HBM read bandwidth a plain
streaming-read kernel achieves over 1 GiB on the same GPU.  The CPU oracle
is timed on a bounded sample of the same workload, on one thread and on all
host cores (whole calls in parallel threads).

`--config m0|m1|m2` (or `--all-moe`) times the mixture-of-experts GEMM fused
with the combine all-to-all instead, on the same principles.

Prints one JSON line per workload (rank 0, N = 1).
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gsa_inputs as gi  # noqa: E402

METRIC = "µs per gemv_allreduce call and achieved HBM GB/s (% of peak), 1 MI355X"
HBM_PEAK_GBPS = 8000.0
DEFAULT_CONFIG = "c4"  # 70B-class MLP down_proj, W=8 N=8192 K=28672 B=4
KERNEL_SOURCE = os.path.join(ROOT, "gemv_shot_all_amd", "csrc", "gemv_allreduce.hip")
MOE_KERNEL_SOURCE = os.path.join(ROOT, "gemv_shot_all_amd", "csrc", "moe_a2a.hip")
MOE_METRIC = "µs per MoE GEMM + combine all-to-all call and achieved HBM GB/s (% of peak), 1 MI355X"


def two_shot_chunk_rows(N, W):
    """Rows of one rank's chunk in the two-shot variant (whole 16-row tiles)."""
    return -(-(-(-N // W)) // 16) * 16


def alg_bytes(W, N, K, B, epilogue=False, two_shot=False, rank=0, slot_bytes=4, out_bytes=4,
              unfused=False):
    """Bytes the method itself must move per call: A_r, x_r, the published
    slot, the W-1 peer slots and out (flags excluded); with the fused
    epilogue also the bias and RMSNorm weight (N fp32 each) and y (bf16).
    Two-shot: the peer slots only over the own chunk's c rows, plus the
    published chunk (c rows) and the N - c rows copied from their owners.
    slot_bytes / out_bytes: element sizes of the slots and of out (4 for
    fp32, 2 for bf16; the two-shot and epilogue calls take fp32).  unfused: the
    epilogue as a second kernel, which reads out back (4 N B more)."""
    Ks = K // W
    if two_shot:
        c = max(0, min(N, (rank + 1) * two_shot_chunk_rows(N, W)) -
                rank * two_shot_chunk_rows(N, W))
        return (2 * N * Ks + 2 * B * Ks + 4 * N * B + 4 * (W - 1) * c * B + 4 * c * B +
                4 * (N - c) * B + 4 * N * B)
    base = (2 * N * Ks + 2 * B * Ks + slot_bytes * N * B + slot_bytes * (W - 1) * N * B +
            out_bytes * N * B)
    return base + (8 * N + 2 * N * B if epilogue else 0) + (4 * N * B if unfused else 0)


def alg_flops(W, N, K, B):
    Ks = K // W
    return 2 * N * Ks * B + (W - 1) * N * B


def kernel_source_digest(path=KERNEL_SOURCE):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def profile_name(cfg, epilogue=False, two_shot=False, slot_dtype="f32", out_dtype="f32",
                 unfused=False):
    """Base name of the committed rocprofv3 summaries for a bench line."""
    variant = ("_rmsnorm_unfused" if unfused else "_rmsnorm" if epilogue else
               "_two_shot" if two_shot else "")
    if slot_dtype != "f32" or out_dtype != "f32":
        variant += f"_slots_{slot_dtype}_out_{out_dtype}"
    return f"gemv_allreduce{variant}_{cfg}"


def traffic_from_profile(cfg, epilogue=False, two_shot=False, name=None, source=KERNEL_SOURCE):
    """HBM bytes per launch from the committed PMC summary for this workload,
    or None if there is none or the kernel source changed since."""
    name = name or profile_name(cfg, epilogue, two_shot)
    path = os.path.join(ROOT, "profiles", name + "_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_digest(source):
        return None
    return float(m_b.group(1))


class Sets:
    """R independent input sets on the device, each with its own symmetric
    buffer (peers published) and output."""

    def __init__(self, d, rotate_bytes, max_sets=None, epilogue=False, two_shot=False,
                 slot_dtype="f32", out_dtype="f32", unfused=False):
        import torch

        import gemv_shot_all_amd as gsa
        self.gsa = gsa
        W, N, K, B = d["W"], d["N"], d["K"], d["B"]
        self.W, self.N, self.K, self.B, self.rank = W, N, K, B, d["rank"]
        self.epilogue = epilogue
        self.unfused = unfused  # the epilogue as a second kernel after the plain call
        self.two_shot = two_shot
        self.slot_bf16 = slot_dtype == "bf16"
        self.out_bf16 = out_dtype == "bf16"
        self.typed = self.slot_bf16 or self.out_bf16
        foot = d["A"].nbytes + d["x"].nbytes + d["slots"].nbytes + 4 * N * B * (2 if two_shot
                                                                                 else 1)
        R = max(1, -(-rotate_bytes // foot) + 1)  # other sets between two uses >= rotate_bytes
        if max_sets:
            R = min(R, max_sets)
        self.R = R
        self.touched = set()  # sets called at least once
        A0 = torch.from_numpy(d["A"].view(np.int16)).cuda()
        x0 = torch.from_numpy(d["x"].view(np.int16)).cuda()
        if self.slot_bf16:
            # the peers' values rounded to bf16 (bits); the own slot is written by the call
            sb = np.zeros(d["slots"].shape, np.uint16)
            for p in range(W):
                if p != self.rank:
                    sb[p] = gi.bf16_bits(d["slots"][p])
            s0 = torch.from_numpy(sb.view(np.int16)).cuda()
        else:
            s0 = torch.from_numpy(d["slots"]).cuda()
        mask = ((1 << W) - 1) & ~(1 << self.rank)
        if two_shot:
            # the other ranks' reduced chunks; the own chunk's rows NaN
            g = gi.make_gathered(N, B, seed=4321, cfg_id=N + B)
            c = two_shot_chunk_rows(N, W)
            g[self.rank * c:(self.rank + 1) * c] = gi.sentinel((B,))
            self.gathered_in = g
            g0 = torch.from_numpy(g).cuda()
        self.A, self.x, self.out, self.bufs = [], [], [], []
        for _ in range(R):
            self.A.append(A0.clone())
            self.x.append(x0.clone())
            if self.out_bf16:
                self.out.append(torch.full((N, B), 0x7FC0, dtype=torch.int16, device="cuda"))
            else:
                self.out.append(torch.full((N, B), float("nan"), dtype=torch.float32,
                                           device="cuda"))
            buf = gsa.SymmBuffer(W, N, B, gsa.GSA_DTYPE_BF16 if self.slot_bf16
                                 else gsa.GSA_DTYPE_F32)
            buf.slots_view().copy_(s0)
            if two_shot:
                buf.gathered_view().copy_(g0)
            buf.reset(mask)
            self.bufs.append(buf)
        self.eps = []
        if epilogue:
            # bias ~ N(0, 0.5), RMSNorm weight ~ N(1, 0.1), eps 1e-5, y in bf16
            rng = np.random.default_rng(1234)
            bias = torch.from_numpy(rng.normal(0, 0.5, N).astype(np.float32)).cuda()
            w = torch.from_numpy(rng.normal(1, 0.1, N).astype(np.float32)).cuda()
            self.epi_tensors = []
            for _ in range(R):
                t = (bias.clone(), w.clone(),
                     torch.empty((N, B), dtype=torch.bfloat16, device="cuda"),
                     torch.empty(B, dtype=torch.float32, device="cuda"))
                self.epi_tensors.append(t)
                self.eps.append(gsa.make_epilogue(t[2], t[0], t[1], 1e-5, t[3]))
        torch.cuda.synchronize()

    def call(self, i):
        j = i % self.R
        self.touched.add(j)
        b = self.bufs[j]
        if self.epilogue and self.unfused:
            self.gsa.gsa_gemv_allreduce(self.A[j], self.x[j], b.slots, b.pad, self.out[j],
                                        self.W, self.rank, self.N, self.K, self.B)
            self.gsa.gsa_bias_rmsnorm(self.out[j], self.N, self.B, self.eps[j])
        elif self.epilogue:
            self.gsa.gsa_gemv_allreduce_rmsnorm(self.A[j], self.x[j], b.slots, b.pad,
                                                self.out[j], self.W, self.rank, self.N, self.K,
                                                self.B, self.eps[j])
        elif self.two_shot:
            self.gsa.gsa_gemv_allreduce_two_shot(self.A[j], self.x[j], b.slots, b.pad,
                                                 b.gathered, self.out[j], self.W, self.rank,
                                                 self.N, self.K, self.B)
        elif self.typed:
            self.gsa.gsa_gemv_allreduce_dtype(
                self.A[j], self.x[j], b.slots, b.pad, self.out[j],
                self.gsa.GSA_DTYPE_BF16 if self.out_bf16 else self.gsa.GSA_DTYPE_F32, self.W,
                self.rank, self.N, self.K, self.B)
        else:
            self.gsa.gsa_gemv_allreduce(self.A[j], self.x[j], b.slots, b.pad, self.out[j],
                                        self.W, self.rank, self.N, self.K, self.B)

    def close(self):
        for b in self.bufs:
            b.close()


def check_consistency(sets):
    """What the timed loop can check without the oracle (that stays in the
    tests and the CPU-baseline leg): every set's out is finite and
    bit-identical to set 0's (the sets hold identical inputs), and in the
    two-shot variant every row outside the own chunk is the other ranks'
    seeded chunk, copied exactly.  Parity against the oracle at these sizes
    is the GPU tests' job."""
    used = sorted(sets.touched)

    def bits(t):
        return t.cpu().numpy().view(np.uint16 if sets.out_bf16 else np.uint32)
    out0 = bits(sets.out[used[0]])
    vals = ((out0.astype(np.uint32) << 16).view(np.float32) if sets.out_bf16
            else out0.view(np.float32))
    ok = bool(np.all(np.isfinite(vals)))
    for j in used[1::max(1, len(used) // 8)]:
        ok = ok and np.array_equal(bits(sets.out[j]), out0)
    if sets.two_shot:
        c = two_shot_chunk_rows(sets.N, sets.W)
        rest = np.ones(sets.N, bool)
        rest[sets.rank * c:(sets.rank + 1) * c] = False
        ok = ok and np.array_equal(out0[rest], sets.gathered_in[rest].view(np.uint32))
    if sets.epilogue:
        y = sets.epi_tensors[used[0]][2].float().cpu().numpy()
        ok = ok and bool(np.all(np.isfinite(y)))
    return ok


class ColdTimer:
    """The timed region's surroundings: a 1 GiB buffer whose read pass
    evicts the input sets from the caches (L2 and the 256 MB Infinity Cache),
    and the bounded spin kernel of libgsa_probe.so that keeps the GPU busy
    while the host queues the graph replay.  The pass only reads (a sum), so
    it leaves no dirty lines whose write-back would land in the timed region
    (a read-and-write pass measured 15.2 against 12.7 us per call for the
    70B-class shape at K = 20: about 50 us of write-back per replay)."""

    def __init__(self, flush_mib):
        import ctypes

        import torch

        from gemv_shot_all_amd import build as gbuild
        if not os.path.exists(gbuild.PROBE_LIBRARY):
            raise RuntimeError(f"{gbuild.PROBE_LIBRARY} is missing; build first")
        self.L = ctypes.CDLL(gbuild.PROBE_LIBRARY)
        self.L.gsa_probe_spin.argtypes = [ctypes.c_uint32, ctypes.c_void_p]
        self.L.gsa_probe_spin.restype = ctypes.c_int
        # flush_mib == 0 (the --warm mode): no eviction pass.
        self.flush_buf = (torch.ones((flush_mib << 20) // 4, dtype=torch.float32,
                                     device="cuda") if flush_mib > 0 else None)
        self.flush_sum = None

    def replay(self, graph, calls, spin_us=20000):
        """Flush, spin, then time one replay of `graph` (holding `calls`
        calls) with HIP events on the current stream.  Returns µs per call."""
        import ctypes

        import torch
        stream = torch.cuda.current_stream()
        if self.flush_buf is not None:
            self.flush_sum = self.flush_buf.sum()
        rc = self.L.gsa_probe_spin(spin_us, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"gsa_probe_spin: {rc}")
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        return 1e3 * ev0.elapsed_time(ev1) / calls

    def close(self):
        self.flush_buf = self.flush_sum = None


def capture(calls_fn):
    """A HIP graph of the calls that calls_fn() enqueues (captured on a side
    stream; a replay runs on the current stream)."""
    import torch
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            calls_fn()
    torch.cuda.synchronize()
    return g


def time_cpu_oracle(d, seconds, threads=1, gathered=None):
    """The oracle as it stands, on whole calls of the same workload, for about
    `seconds` of wall time on `threads` threads (each runs whole calls; the
    C oracle runs without the Python lock).  With `gathered` a call is the
    two-shot one: the fp64 GEMV, its fp32 rounding into the own slot, then
    the oracle's two-shot step.  Returns (wall µs per call, calls)."""
    import threading

    import oracle
    o = oracle.load()

    def one_call():
        if gathered is None:
            o.gemv_allreduce(d["A"], d["x"], d["slots"], d["rank"])
        else:
            y64, _ = o.gemv(d["A"], d["x"])
            slots = d["slots"].copy()
            slots[d["rank"]] = y64.astype(np.float32)
            o.two_shot(slots, gathered, d["rank"])
    t0 = time.perf_counter()
    one_call()
    one = time.perf_counter() - t0
    n = max(1, int(seconds / max(one, 1e-6)))  # calls per thread
    def work():
        for _ in range(n):
            one_call()
    ts = [threading.Thread(target=work) for _ in range(threads)]
    t0 = time.perf_counter()
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    el = time.perf_counter() - t0
    return 1e6 * el / (n * threads), n * threads


def host_threads():
    """Threads the host offers this process (at most 16, the CPU share of one
    GPU on a shared node)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def hbm_read_probe(gib=1, launches=20):
    """Best HBM read bandwidth (GB/s) of the plain streaming-read kernel of
    libgsa_probe.so over `gib` GiB, over a few grid sizes."""
    import ctypes

    import torch

    from gemv_shot_all_amd import build as gbuild
    if not os.path.exists(gbuild.PROBE_LIBRARY):
        return None
    L = ctypes.CDLL(gbuild.PROBE_LIBRARY)
    L.gsa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                 ctypes.c_int, ctypes.c_void_p]
    L.gsa_probe_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = None
    for grid in (256, 512, 1024, 2048, 4096, 8192):
        def launch():
            rc = L.gsa_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid,
                                  ctypes.c_void_p(stream.cuda_stream))
            if rc != 0:
                raise RuntimeError(f"gsa_probe_read: {rc}")
        launch()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(launches):
            launch()
        ev1.record(stream)
        torch.cuda.synchronize()
        gbps = nbytes * launches / (ev0.elapsed_time(ev1) * 1e-3) / 1e9
        best = gbps if best is None else max(best, gbps)
    del buf, sink
    return round(best, 1)


def run_config(cfg, args):
    import torch

    d = gi.make_inputs(cfg, seed=args.seed, rank=0)
    W, N, K, B = d["W"], d["N"], d["K"], d["B"]
    sets = Sets(d, args.rotate_mib << 20 if not args.warm else 1, args.max_sets, args.epilogue,
                args.two_shot, args.slot_dtype, args.out_dtype, args.epilogue_unfused)
    timer = ColdTimer(args.flush_mib if not args.warm else 0)
    try:
        # Warm-up: exactly args.warmup untimed calls.
        for i in range(args.warmup):
            sets.call(i)
        torch.cuda.synchronize()

        # Timed region: K calls continuing the rotation, in one graph replay
        # after a cache-evicting pass (see the module docstring).
        K_ = args.steps
        g = capture(lambda: [sets.call(args.warmup + j) for j in range(K_)])
        us_per_call = timer.replay(g, K_)
        consistent = check_consistency(sets)

        # For reference, after the timed region: the same replay again (cold
        # again; shows whether the first replay of a graph costs extra), host-
        # issued launches, and a warm pass over one resident set (its inputs
        # stay in the Infinity Cache and L2: not HBM).
        second_us = timer.replay(g, K_)
        torch.cuda.synchronize()
        t_e0 = time.perf_counter()
        for j in range(K_):
            sets.call(args.warmup + j)
        torch.cuda.synchronize()
        eager_us = 1e6 * (time.perf_counter() - t_e0) / K_
        gw = capture(lambda: [sets.call(0) for _ in range(K_)])
        gw.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        gw.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        warm_us = 1e3 * ev0.elapsed_time(ev1) / K_
        consistent = consistent and check_consistency(sets)
        del g, gw
    finally:
        gathered_in = getattr(sets, "gathered_in", None)
        timer.close()
        sets.close()

    nbytes = alg_bytes(W, N, K, B, args.epilogue, args.two_shot, unfused=args.epilogue_unfused,
                       slot_bytes=2 if args.slot_dtype == "bf16" else 4,
                       out_bytes=2 if args.out_dtype == "bf16" else 4)
    achieved = nbytes / (us_per_call * 1e-6) / 1e9
    traffic = traffic_from_profile(cfg, name=profile_name(cfg, args.epilogue, args.two_shot,
                                                          args.slot_dtype, args.out_dtype,
                                                          unfused=args.epilogue_unfused))
    line = {
        "metric": METRIC,
        "value": round(us_per_call, 4),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call / 1e3, 7),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": gi.CONFIGS[cfg]["name"], "id": cfg, "W": W, "rank": 0, "N": N,
            "K": K, "B": B, "accumulate": "f32",
            "inputs": ("cold: %d resident sets rotated, %d MiB read between the warm-up "
                       "and the timed replay" % (sets.R, args.flush_mib))
                      if not args.warm else "warm: one set (Infinity-Cache resident, not HBM)",
            "timing": "hipGraph replay of K calls, HIP events on the launch stream, between "
                      "two device syncs",
            "untimed_calls_before_timed_region": args.warmup,
            "epilogue": ("bias + RMSNorm over rows (eps 1e-5), y in bf16, as a second kernel "
                         "(gsa_bias_rmsnorm) after the plain call" if args.epilogue_unfused else
                         "bias + RMSNorm over rows (eps 1e-5), y in bf16" if args.epilogue
                         else "none"),
            "all_reduce": "two-shot" if args.two_shot else "one-shot",
            "slots": args.slot_dtype, "out": args.out_dtype,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": nbytes,
            "launch_us_mean": round(us_per_call, 4),
        },
        "extra": {
            "second_cold_replay_us_per_call": round(second_us, 4),
            "eager_us_per_call": round(eager_us, 4),
            "warm_us_per_call": round(warm_us, 4),
            "sets_consistent": consistent,
            "alg_flops_per_call": alg_flops(W, N, K, B),
        },
    }
    if args.cpu_seconds > 0:
        threads = host_threads()
        g = gathered_in if args.two_shot else None
        st_us, st_calls = time_cpu_oracle(d, args.cpu_seconds / 2, threads=1, gathered=g)
        mt_us, mt_calls = time_cpu_oracle(d, args.cpu_seconds / 2, threads=threads, gathered=g)
        line["cpu_baseline"] = {
            "value": round(mt_us, 2), "unit": "us/call", "cores": threads, "kind": "oracle",
            "sample": f"{mt_calls} whole calls of the {cfg} workload (fp64) on {threads} "
                      f"threads in parallel, wall time per call; host: {os.cpu_count()} "
                      f"logical CPUs, {cpu_model()}",
            "single_thread_us_per_call": round(st_us, 2),
            "single_thread_calls": st_calls,
        }
    else:
        line["cpu_baseline"] = None
    return line


def moe_alg_bytes(d):
    """Bytes the MoE call must move: the weights of every local expert that
    has tokens (2 H F each), its dispatched rows (2 F per token) and the
    result rows pushed to the combine buffers (4 H per token); split tables
    and flags excluded."""
    M = d["length"].sum(axis=1)
    H, F = d["H"], d["F"]
    return int((M > 0).sum()) * 2 * H * F + int(M.sum()) * (2 * F + 4 * H)


class MoeSets:
    """R independent MoE input sets on the device, each with its own combine
    buffers and pads (peers published)."""

    def __init__(self, d, rotate_bytes, max_sets=None):
        import torch

        import gemv_shot_all_amd as gsa
        self.gsa, self.d = gsa, d
        foot = d["Wd"].nbytes + d["X"].nbytes + d["bufs"].nbytes
        R = max(1, -(-rotate_bytes // foot) + 1)  # other sets between two uses >= rotate_bytes
        if max_sets:
            R = min(R, max_sets)
        self.R = R
        self.touched = set()  # sets called at least once
        Wd0 = torch.from_numpy(d["Wd"].view(np.int16)).cuda()
        X0 = torch.from_numpy(d["X"].view(np.int16)).cuda()
        b0 = torch.from_numpy(d["bufs"]).cuda()
        splits = torch.from_numpy(np.concatenate([d["length"].ravel(),
                                                  d["in_off"].ravel()]).astype(np.int32)).cuda()
        dst = torch.from_numpy(d["dst_off"].astype(np.int32).ravel()).cuda()
        W, rank = d["W"], d["rank"]
        mask = ((1 << W) - 1) & ~(1 << rank)
        self.Wd, self.X, self.splits, self.dst, self.bufs = [], [], [], [], []
        for _ in range(R):
            self.Wd.append(Wd0.clone())
            self.X.append(X0.clone())
            self.splits.append(splits.clone())
            self.dst.append(dst.clone())
            buf = gsa.A2ABuffer(W, d["ne"], d["H"], d["rows_out"])
            buf.bufs_view().copy_(b0)
            buf.reset(mask)
            self.bufs.append(buf)
        del Wd0
        torch.cuda.synchronize()

    def call(self, i):
        j = i % self.R
        self.touched.add(j)
        d, b = self.d, self.bufs[j]
        self.gsa.gsa_moe_gemm_all_to_all(self.X[j], self.Wd[j], self.splits[j], self.dst[j],
                                         b.bufs, b.pads, d["W"], d["rank"], d["ne"], d["H"],
                                         d["F"], d["rows_in"], d["rows_out"])

    def check_consistency(self):
        """Every called set's combine buffers bit-identical to the first
        one's, finite where the combine writes; every set's status OK."""
        used = sorted(self.touched)
        out0 = self.bufs[used[0]].bufs_view().cpu().numpy()
        ok = bool(np.all(np.isfinite(out0)))
        for j in range(self.R):
            ok = ok and self.bufs[j].status(self.d["rank"]) == (0, -1, -1)
        for j in used[1::max(1, len(used) // 8)]:
            ok = ok and np.array_equal(self.bufs[j].bufs_view().cpu().numpy().view(np.uint32),
                                       out0.view(np.uint32))
        return ok

    def close(self):
        for b in self.bufs:
            b.close()


def time_cpu_oracle_moe(d, seconds, threads=1):
    """The oracle's moe_combine on whole calls, as time_cpu_oracle."""
    import threading

    import oracle
    o = oracle.load()

    def one_call():
        o.moe_combine(d["X"], d["Wd"], d["length"], d["in_off"], d["dst_off"], d["W"],
                      d["rows_out"])
    t0 = time.perf_counter()
    one_call()
    one = time.perf_counter() - t0
    n = max(1, int(seconds / max(one, 1e-6)))

    def work():
        for _ in range(n):
            one_call()
    ts = [threading.Thread(target=work) for _ in range(threads)]
    t0 = time.perf_counter()
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    el = time.perf_counter() - t0
    return 1e6 * el / (n * threads), n * threads


def run_moe_config(cfg, args):
    import torch

    d = gi.make_moe_inputs(cfg, seed=args.seed, rank=0)
    sets = MoeSets(d, args.rotate_mib << 20 if not args.warm else 1, args.max_sets)
    timer = ColdTimer(args.flush_mib if not args.warm else 0)
    try:
        for i in range(args.warmup):
            sets.call(i)
        torch.cuda.synchronize()
        K_ = args.steps
        g = capture(lambda: [sets.call(args.warmup + j) for j in range(K_)])
        us_per_call = timer.replay(g, K_)
        consistent = sets.check_consistency()
        second_us = timer.replay(g, K_)
        consistent = consistent and sets.check_consistency()
        del g
    finally:
        R = sets.R
        timer.close()
        sets.close()
    nbytes = moe_alg_bytes(d)
    achieved = nbytes / (us_per_call * 1e-6) / 1e9
    name = f"moe_gemm_all_to_all_{cfg}"
    c = gi.MOE_CONFIGS[cfg]
    M = d["length"].sum(axis=1)
    line = {
        "metric": MOE_METRIC,
        "value": round(us_per_call, 4),
        "unit": "us/call",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us_per_call / 1e3, 7),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": c["name"], "id": cfg, "W": d["W"], "rank": 0, "ne": d["ne"],
            "H": d["H"], "F": d["F"], "top_k": c["top_k"], "tokens_per_rank": c["T"],
            "tokens_received": int(M.sum()), "experts_with_tokens": int((M > 0).sum()),
            "accumulate": "f32", "out": "f32",
            "inputs": ("cold: %d resident sets rotated, %d MiB read between the warm-up "
                       "and the timed replay" % (R, args.flush_mib))
                      if not args.warm else "warm: one set (Infinity-Cache resident, not HBM)",
            "timing": "hipGraph replay of K calls, HIP events on the launch stream, between "
                      "two device syncs",
            "untimed_calls_before_timed_region": args.warmup,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic_from_profile(cfg, name=name, source=MOE_KERNEL_SOURCE),
            "alg_bytes_per_launch": nbytes,
            "launch_us_mean": round(us_per_call, 4),
        },
        "extra": {
            "second_cold_replay_us_per_call": round(second_us, 4),
            "sets_consistent": consistent,
            "alg_flops_per_call": int(2 * d["H"] * d["F"] * M.sum()),
        },
    }
    if args.cpu_seconds > 0:
        threads = host_threads()
        st_us, st_calls = time_cpu_oracle_moe(d, args.cpu_seconds / 2, threads=1)
        mt_us, mt_calls = time_cpu_oracle_moe(d, args.cpu_seconds / 2, threads=threads)
        line["cpu_baseline"] = {
            "value": round(mt_us, 2), "unit": "us/call", "cores": threads, "kind": "oracle",
            "sample": f"{mt_calls} whole calls of the {cfg} workload (fp64) on {threads} "
                      f"threads in parallel, wall time per call; host: {os.cpu_count()} "
                      f"logical CPUs, {cpu_model()}",
            "single_thread_us_per_call": round(st_us, 2),
            "single_thread_calls": st_calls,
        }
    else:
        line["cpu_baseline"] = None
    return line


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", default=DEFAULT_CONFIG,
                   choices=sorted(gi.CONFIGS) + sorted(gi.MOE_CONFIGS),
                   help="a GEMV + AllReduce workload, or m0/m1/m2 for the MoE GEMM + "
                        "combine all-to-all")
    p.add_argument("--all", action="store_true", help="one line per workload")
    p.add_argument("--all-moe", action="store_true", help="one line per MoE workload")
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--rotate-mib", type=int, default=1024,
                   help="total size of the rotated input sets (MiB)")
    p.add_argument("--max-sets", type=int, default=None)
    p.add_argument("--flush-mib", type=int, default=1024,
                   help="size of the buffer read between the warm-up and the "
                        "timed replay (MiB)")
    p.add_argument("--warm", action="store_true", help="one resident set (cache-warm)")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="CPU-oracle wall-time budget, split between one thread and all "
                        "host threads (0 = skip)")
    p.add_argument("--epilogue", action="store_true",
                   help="time gsa_gemv_allreduce_rmsnorm (bias + RMSNorm, y in bf16) instead")
    p.add_argument("--epilogue-unfused", action="store_true",
                   help="time the plain call followed by gsa_bias_rmsnorm (the same epilogue "
                        "as a second kernel) in the same graph")
    p.add_argument("--two-shot", action="store_true",
                   help="time gsa_gemv_allreduce_two_shot (reduce the own chunk, copy the "
                        "others) instead")
    p.add_argument("--slot-dtype", choices=("f32", "bf16"), default="f32",
                   help="element type of the slots (bf16: published and summed as bf16 "
                        "values, fp32 accumulation)")
    p.add_argument("--out-dtype", choices=("f32", "bf16"), default="f32",
                   help="element type of out")
    p.add_argument("--no-probe", action="store_true",
                   help="skip the 1 GiB streaming-read bandwidth reference")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="also run a plain device copy of this many MiB five times "
                        "(reference kernel for scaling HBM byte counters)")
    args = p.parse_args()
    if args.epilogue_unfused:
        args.epilogue = True
    if args.epilogue and args.two_shot:
        p.error("--epilogue and --two-shot are separate entry points; pick one")
    if (args.epilogue or args.two_shot) and (args.slot_dtype != "f32" or args.out_dtype != "f32"):
        p.error("the epilogue and two-shot calls take fp32 slots and out")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU's share of the operator on one MI355X; "
              "multi-GPU runs are not implemented (each rank would run this same "
              "kernel on its own shard).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (MI355X)", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration_mib:
        # A plain streaming kernel that reads and writes exactly n bytes
        # (float32 multiply by one), under a kernel name of its own.
        n = args.copy_calibration_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    probe = hbm_read_probe() if not args.no_probe else None
    cfgs = list(gi.CONFIGS) if args.all else [] if args.all_moe else [args.config]
    if args.all_moe:
        cfgs += list(gi.MOE_CONFIGS)
    for cfg in cfgs:
        line = run_moe_config(cfg, args) if cfg in gi.MOE_CONFIGS else run_config(cfg, args)
        line["extra"]["hbm_read_probe_GBps"] = probe
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
