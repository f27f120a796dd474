"""Host checks of the GEMM+ReduceScatter work queues (no GPU): the kernel's own
task decode (gemm_rs_geom.h) holds every (destination, tile, source) task once
per queue, and the receiver's task of each tile (source == destination, the one
that waits and adds) after the W - 1 tasks it waits for (the deadlock-freedom
argument); the argument checks reject what the kernel cannot run."""
import pytest

import moe_all2all_combine_amd as ra2a

SHAPES = [
    # W, m, K, N
    (8, 8192, 896, 4096),
    (8, 512, 512, 512),
    (3, 300, 72, 200),
    (3, 300, 72, 202),
    (1, 5, 8, 8),
    (2, 2, 8, 3000),
    (16, 2048, 64, 264),
    (5, 5 * 700, 16, 1000),
    (8, 8 * 257, 8, 257),
    (2, 2 * 2048, 64, 2304),   # 72 tiles per destination: three queue blocks, the last ragged
    (3, 3 * 4096, 8, 4096),    # 256 tiles per destination: eight full blocks
]


@pytest.mark.parametrize("W,m,K,N", SHAPES)
@pytest.mark.parametrize("num_xcd", [8, 3, 1])
def test_queues_hold_every_task_once_and_waits_point_backwards(W, m, K, N, num_xcd):
    n = ra2a.debug_gemm_rs_plan(W, m, K, N, num_xcd)
    tiles = -(-(m // W) // 256) * -(-N // 256)
    groups = min(num_xcd, 8)
    assert n == tiles * W * -(-W // groups)


def test_sizes():
    # the receive area holds W slots of one whole 256 x 256 tile per output tile
    t, q, p = ra2a.gemm_rs_sizes(3, 300, 72, 202)
    assert (t, q, p) == (1 * 1 * 3, ra2a.QUEUE_SLOTS, 3 * 1 * 256 * 256 * 4)
    t, q, p = ra2a.gemm_rs_sizes(8, 8192, 896, 4096)
    assert (t, q, p) == (4 * 16 * 8, ra2a.QUEUE_SLOTS, 8 * 1024 * 4096 * 4)
    t, q, p = ra2a.gemm_rs_sizes(8, 8192, 896, 4096, ra2a.RS_BF16_PARTIALS)
    assert (t, q, p) == (4 * 16 * 8, ra2a.QUEUE_SLOTS, 8 * 1024 * 4096 * 2)
    # the sync and reset flags do not change the sizes
    assert ra2a.gemm_rs_sizes(8, 8192, 896, 4096, ra2a.RS_AGENT_SYNC | ra2a.RS_SKIP_RESET)[2] == \
        8 * 1024 * 4096 * 4


def test_unknown_flags_rejected():
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.gemm_rs_sizes(8, 8192, 896, 4096, 8)
    assert e.value.code == ra2a.EINVAL


def test_f32_partials_hit_the_4gib_limit_first():
    # 8 slots of 32 x 96 tiles of 256 x 256: 3.2 GB in bf16, 6.4 GB in fp32
    ra2a.gemm_rs_sizes(8, 8 * 8000, 8, 24576, ra2a.RS_BF16_PARTIALS)
    with pytest.raises(ra2a.Ra2aError):
        ra2a.gemm_rs_sizes(8, 8 * 8000, 8, 24576)


@pytest.mark.parametrize("args", [(3, 100, 8, 8),      # m not divisible by W
                                  (2, 8, 12, 8),       # K not a multiple of 8
                                  (0, 8, 8, 8), (2, 0, 8, 8), (2, 8, 8, 0),
                                  (8, 8 * 20000, 8, 8192)])  # receive area above 4 GiB
def test_rejected_shapes(args):
    with pytest.raises(ra2a.Ra2aError) as e:
        ra2a.gemm_rs_sizes(*args)
    assert e.value.code == ra2a.EINVAL


def test_k_limit_of_32_bit_operand_offsets():
    """A tile's 256 operand rows of K bf16 are addressed with 32-bit offsets: the
    largest K accepted keeps 256 * K * 2 bytes below 4 GiB (less a 64 KiB margin)."""
    ok_k = (1 << 23) - 256           # 256 * K * 2 = 2^32 - 2^17
    assert ra2a.gemm_rs_sizes(1, 1, ok_k, 8)[0] == 1
    for K in ((1 << 23) - 128, 1 << 23):
        with pytest.raises(ra2a.Ra2aError) as e:
            ra2a.gemm_rs_sizes(1, 1, K, 8)
        assert e.value.code == ra2a.EINVAL
