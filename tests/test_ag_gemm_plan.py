"""Host checks of the AllGather+GEMM work queues (``ra2a_debug_ag_gemm_plan``):
every AllGather part and GEMM tile queued exactly once, the parts covering each
shard's rows once without straddling a signalled tile, and every GEMM tile
queued after all parts of the tiles it waits for -- the kernel's deadlock-
freedom argument.  No GPU needed."""
import pytest

import moe_all2all_combine_amd as ra2a


@pytest.mark.parametrize("W,rank,m_local,K,N,tile_rows", [
    (8, 0, 1024, 7168, 4096, 128),     # the AllGather+GEMM workload
    (8, 5, 1024, 7168, 4096, 128),
    (3, 1, 300, 72, 200, 100), (1, 0, 5, 8, 8, 1), (8, 3, 1000, 64, 264, 1000),
    (16, 2, 777, 40, 520, 64), (2, 0, 256, 16, 256, 256), (5, 4, 513, 8, 8, 129),
    (4, 0, 2048, 8, 16, 7), (9, 8, 64, 4096, 8, 512), (8, 0, 257, 7168, 256, 300),
])
@pytest.mark.parametrize("num_xcd", [8, 1, 3, 4])
def test_plan_queues(W, rank, m_local, K, N, tile_rows, num_xcd):
    n = ra2a.debug_ag_gemm_plan(W, rank, m_local, K, N, tile_rows, num_xcd)
    assert n > 0


def test_plan_task_count_of_the_workload():
    # 8 tiles of 128 rows x 7168: 1.75 MiB each in 13 parts of <= 10 rows; 4 x 16 GEMM tiles
    assert ra2a.debug_ag_gemm_plan(8, 0, 1024, 7168, 4096, 128, 8) == 8 * 13 + 4 * 16


@pytest.mark.parametrize("bad", [
    dict(W=0), dict(rank=8), dict(rank=-1), dict(m_local=0), dict(K=12), dict(N=4),
    dict(tile_rows=0),
    dict(K=1 << 23),  # 256 rows x K x 2 bytes reach 4 GiB: past the tile's 32-bit offsets
])
def test_plan_rejects_bad_arguments(bad):
    args = dict(W=8, rank=0, m_local=64, K=64, N=64, tile_rows=16)
    args.update(bad)
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.debug_ag_gemm_plan(args["W"], args["rank"], args["m_local"], args["K"], args["N"],
                                args["tile_rows"])
    assert e.value.code == ra2a.EINVAL


def test_signal_slot_counts():
    assert ra2a.ag_gemm_signal_slots(8, 1024, 128) == (64, 64, ra2a.QUEUE_SLOTS)
    assert ra2a.ag_gemm_signal_slots(3, 300, 100) == (9, 9, ra2a.QUEUE_SLOTS)
    assert ra2a.ag_gemm_signal_slots(2, 5, 1000) == (2, 2, ra2a.QUEUE_SLOTS)  # one tile per shard


def test_largest_k_within_32_bit_operand_offsets():
    assert ra2a.debug_ag_gemm_plan(8, 0, 64, (1 << 23) - 256, 64, 16) > 0
