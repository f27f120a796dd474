"""GPU tests of the one-sided primitives through the C ABI: put_with_signal,
put, get, signal_op, wait_signal (all six predicates), signal_reset and the
bounded wait's time-out path (forced from the host with a tiny time limit and
a value the host never writes, so every kernel still exits normally)."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import moe_all2all_combine_amd as ra2a  # noqa: E402
import oracle  # noqa: E402

from combine_harness import say  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture
def heap():
    h = ra2a.SymmHeap(4, 8 << 20)
    yield h
    h.close()


def sig_value(heap, off, rank):
    return int(heap.view(off, (16,), torch.int64, rank)[0].item())


def test_put_with_signal_example_shape(heap):
    """4096 fp16 values from rank 0 to rank 1 with SET 1; rank 1 waits EQ 1 on another
    stream, then reads the data (the RFC's first usage example, section 十四)."""
    say("[case] put_with_signal 4096 f16 SET 1 -> rank 1, wait EQ 1")
    data = heap.alloc(4096 * 2)
    sig = heap.alloc(128)
    ra2a.signal_reset(heap.handle, heap.ptr(sig), 1)
    src = torch.randn(4096, device="cuda").to(torch.float16)
    consumer = torch.cuda.Stream()
    producer = torch.cuda.Stream()
    torch.cuda.synchronize()
    # producer first: should both streams share one hardware queue, the put still runs
    ra2a.put_with_signal(heap.handle, heap.ptr(data), src.data_ptr(), 4096 * 2, heap.ptr(sig), 1,
                         ra2a.SIG_SET, 1, producer)
    ra2a.wait_signal(heap.handle, heap.ptr(sig, 1), 1, ra2a.CMP_EQ, consumer)
    with torch.cuda.stream(consumer):
        got = heap.view(data, (4096,), torch.int16, 1).clone()
    torch.cuda.synchronize()
    assert ra2a.check(heap.handle) == ra2a.OK, ra2a.last_error()
    assert torch.equal(got, src.view(torch.int16))
    assert sig_value(heap, sig, 1) == 1
    assert sig_value(heap, sig, 0) == 0


@pytest.mark.parametrize("nbytes", [0, 1, 13, 4096, 300 * 1024 + 7, 3 << 20])
def test_put_add_and_get(heap, nbytes):
    say(f"[case] put_with_signal ADD nbytes={nbytes}")
    dst = heap.alloc(max(nbytes, 1))
    sig = heap.alloc(128)
    ra2a.signal_reset(heap.handle, heap.ptr(sig), 1)
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (max(nbytes, 1),), dtype=torch.uint8, generator=g).cuda()
    for target in range(4):
        ra2a.put_with_signal(heap.handle, heap.ptr(dst), src.data_ptr(), nbytes, heap.ptr(sig), 5,
                             ra2a.SIG_ADD, target)
        ra2a.signal_op(heap.handle, heap.ptr(sig), 2, ra2a.SIG_ADD, target)
    back = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    ra2a.get(heap.handle, back.data_ptr(), heap.ptr(dst), nbytes, 3)
    torch.cuda.synchronize()
    for target in range(4):
        assert sig_value(heap, sig, target) == oracle.signal_apply(oracle.signal_apply(0, 5, "add"),
                                                                   2, "add")
        if nbytes:
            assert torch.equal(heap.view(dst, (nbytes,), torch.uint8, target), src[:nbytes])
    if nbytes:
        assert torch.equal(back[:nbytes], src[:nbytes])


def test_put_alone(heap):
    dst = heap.alloc(1 << 20)
    src = torch.arange(1 << 18, dtype=torch.int32, device="cuda")
    ra2a.put(heap.handle, heap.ptr(dst), src.data_ptr(), 1 << 20, 2)
    torch.cuda.synchronize()
    assert torch.equal(heap.view(dst, (1 << 18,), torch.int32, 2), src)


@pytest.mark.parametrize("op", ["eq", "ne", "gt", "ge", "lt", "le"])
def test_wait_predicates_that_hold_return(heap, op):
    """A wait whose predicate holds returns; the value is not consumed."""
    sig = heap.alloc(128)
    ra2a.signal_reset(heap.handle, heap.ptr(sig), 1)
    value = 7
    ra2a.signal_op(heap.handle, heap.ptr(sig), value, ra2a.SIG_SET, 0)
    code = {"eq": ra2a.CMP_EQ, "ne": ra2a.CMP_NE, "gt": ra2a.CMP_GT, "ge": ra2a.CMP_GE,
            "lt": ra2a.CMP_LT, "le": ra2a.CMP_LE}[op]
    # pick a comparison value for which the oracle says the predicate holds
    cmp_value = next(c for c in (7, 6, 8) if oracle.compare(value, c, op))
    say(f"[case] wait {op} {cmp_value} on {value}")
    for _ in range(3):
        ra2a.wait_signal(heap.handle, heap.ptr(sig), cmp_value, code)
    torch.cuda.synchronize()
    assert ra2a.check(heap.handle) == ra2a.OK
    assert sig_value(heap, sig, 0) == value


def test_wait_times_out_and_reports(heap):
    """A value nobody writes: the bounded wait gives up, check() reports it once."""
    sig = heap.alloc(128)
    ra2a.signal_reset(heap.handle, heap.ptr(sig), 1)
    ra2a.set_spin_timeout(heap.handle, 2000)  # 2 ms
    say("[case] wait EQ 5 on a signal that stays 0, 2 ms limit")
    ra2a.wait_signal(heap.handle, heap.ptr(sig), 5, ra2a.CMP_EQ)
    torch.cuda.synchronize()
    assert ra2a.check(heap.handle) == ra2a.ETIMEOUT
    assert ra2a.check(heap.handle) == ra2a.OK
    ra2a.set_spin_timeout(heap.handle, 0)


def test_signal_reset_every_slice(heap):
    sig = heap.alloc(10 * 128)
    for r in range(4):
        heap.view(sig, (10, 16), torch.int64, r).fill_(-1)
    ra2a.signal_reset(heap.handle, heap.ptr(sig), 10)
    torch.cuda.synchronize()
    for r in range(4):
        v = heap.view(sig, (10, 16), torch.int64, r)
        assert (v[:, 0] == 0).all() and (v[:, 1:] == -1).all()


def test_library_owned_heap():
    h = ra2a.symm_heap_create(3, 1 << 20)
    try:
        base, stride, world = ra2a.symm_heap_info(h)
        assert world == 3 and stride == 2 << 20 and base % 256 == 0
        off = ra2a.symm_malloc(h, 4096)
        src = torch.arange(1024, dtype=torch.int32, device="cuda")
        ra2a.put(h, base + off, src.data_ptr(), 4096, 2)
        back = torch.empty_like(src)
        ra2a.get(h, back.data_ptr(), base + off, 4096, 2)
        torch.cuda.synchronize()
        assert torch.equal(back, src)
    finally:
        ra2a.symm_heap_destroy(h)


@pytest.mark.parametrize("nbytes", [(100 << 20) + 48, (33 << 20) + 3])
def test_wide_put_loops_over_segments(nbytes):
    """Puts large enough that each of the 2048 workgroups copies several segments
    (16-byte vectors, and 1-byte vectors for an odd size), with a ragged tail."""
    say(f"[case] wide put nbytes={nbytes}")
    h = ra2a.SymmHeap(2, nbytes + (1 << 20))
    try:
        dst = h.alloc(nbytes)
        g = torch.Generator(device="cuda").manual_seed(nbytes % 1000)
        src = torch.randint(0, 256, (nbytes + 1,), dtype=torch.uint8, generator=g, device="cuda")
        h.view(dst, (nbytes,), torch.uint8, 1).fill_(0)
        off = nbytes % 2  # odd sizes also start one byte in: 1-byte vectors
        ra2a.put(h.handle, h.ptr(dst), src.data_ptr() + off, nbytes, 1)
        torch.cuda.synchronize()
        assert ra2a.check(h.handle) == ra2a.OK
        assert torch.equal(h.view(dst, (nbytes,), torch.uint8, 1), src[off:off + nbytes])
    finally:
        h.close()
