"""Host-side helpers of bench.py (no GPU): algorithmic byte counts and the
two-shot chunk size, checked against hand counts and the oracle."""
import sys

import bench
import gsa_inputs as gi
import oracle


def test_alg_bytes_one_shot_by_hand():
    # o_proj shape: A 4096 x 512 bf16, x 512 bf16, own slot 4096 fp32, 7 peer
    # slots, out 4096 fp32
    assert bench.alg_bytes(8, 4096, 4096, 1) == (4096 * 512 * 2 + 512 * 2 + 4096 * 4 +
                                                 7 * 4096 * 4 + 4096 * 4)
    # the epilogue adds bias and weight (fp32) and a bf16 y
    assert (bench.alg_bytes(8, 4096, 4096, 1, epilogue=True) -
            bench.alg_bytes(8, 4096, 4096, 1)) == 8 * 4096 + 2 * 4096


def test_alg_bytes_bf16_slots_and_out_by_hand():
    # 70B-class shape with bf16 slots and bf16 out: A 8192 x 3584 bf16, x 4 x
    # 3584 bf16, own slot, 7 peer slots and out at 2 bytes per element
    assert bench.alg_bytes(8, 8192, 28672, 4, slot_bytes=2, out_bytes=2) == (
        8192 * 3584 * 2 + 4 * 3584 * 2 + 8192 * 4 * 2 + 7 * 8192 * 4 * 2 + 8192 * 4 * 2)
    # bf16 out alone saves 2 bytes per output element
    assert (bench.alg_bytes(8, 4096, 4096, 1) - bench.alg_bytes(8, 4096, 4096, 1, out_bytes=2)
            == 2 * 4096)


def test_alg_bytes_unfused_epilogue_by_hand():
    # the epilogue as a second kernel reads out back: 4 N B more than fused
    assert (bench.alg_bytes(8, 4096, 4096, 1, epilogue=True, unfused=True) -
            bench.alg_bytes(8, 4096, 4096, 1, epilogue=True)) == 4 * 4096
    assert bench.profile_name("c2", epilogue=True, unfused=True) == "gemv_allreduce_rmsnorm_unfused_c2"


def test_alg_bytes_two_shot_by_hand():
    # rank 0 of 8 owns 512 rows: 7 peers x 512 rows, its 512 published rows,
    # 3584 copied rows
    base = 4096 * 512 * 2 + 512 * 2 + 4096 * 4 + 4096 * 4
    assert bench.alg_bytes(8, 4096, 4096, 1, two_shot=True) == (
        base + 7 * 512 * 4 + 512 * 4 + 3584 * 4)


def test_two_shot_chunk_rows_matches_oracle():
    o = oracle.load()
    for N in (1, 15, 16, 17, 1000, 4096, 4097, 8192, 96005):
        for W in (1, 2, 3, 4, 7, 8):
            assert bench.two_shot_chunk_rows(N, W) == o.two_shot_chunk_rows(N, W), (N, W)


def test_moe_alg_bytes_by_hand():
    d = gi.make_moe_inputs("m0", seed=0, rank=0)
    M = d["length"].sum(axis=1)
    want = sum(2 * d["H"] * d["F"] for m in M if m > 0) + int(M.sum()) * (2 * d["F"] + 4 * d["H"])
    assert bench.moe_alg_bytes(d) == want


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr(sys, "argv", ["bench.py", "--gpus", "2"])
    try:
        bench.main()
        raise AssertionError("bench.main() returned")
    except SystemExit as e:
        assert e.code == 2
    assert "one GPU" in capsys.readouterr().err
