"""Pins of the signal-protocol model: exhaustive interleavings, seeded schedules,
closed-form final states, and negative controls that each turn one rule off.

The negative controls are the failure modes the pages warn about: a launch
without the host's signal reset ("Host Side Modifications"), a signal issued
before the data is fenced (fence-before-signal in the RFC's put_with_signal),
a producer that reuses a ring slot without waiting for the hand-back, and a
producer piece that never arrives.
"""
import pytest

import oracle
from oracle.protocol import ADD, SET, ProtocolSpec, explore_all, run_random


def ok_spec(protocol, **kw):
    base = dict(W=2, nbs=3, nstreams=1, R=1, protocol=protocol, n_producers=2, n_consumers=2)
    base.update(kw)
    return ProtocolSpec(**base)


@pytest.mark.parametrize("protocol", [ADD, SET])
def test_exhaustive_no_violation_no_deadlock(protocol):
    spec = ok_spec(protocol, nbs=2)
    states, violations, deadlock = explore_all(spec)
    assert states > 100
    assert violations == []
    assert not deadlock


@pytest.mark.parametrize("protocol", [ADD, SET])
@pytest.mark.parametrize("R", [1, 2, 4])
def test_seeded_schedules_match_closed_forms(protocol, R):
    spec = ok_spec(protocol, W=3, nbs=5, nstreams=2, R=R, n_producers=3, n_consumers=2)
    want_sig = oracle.protocol.expected_final_signals(spec)
    want_cred = oracle.protocol.expected_final_credits(spec)
    for seed in range(200):
        out = run_random(spec, seed)
        assert out.completed and out.violations == []
        assert out.signals == want_sig
        assert out.credits == want_cred
        assert all(v == k[2] for k, v in out.out.items())


def test_closed_form_counts():
    spec = ok_spec(ADD, W=8, nbs=8, nstreams=16, R=2)
    sig = oracle.protocol.expected_final_signals(spec)
    assert len(sig) == 8 * 8 * 16 and set(sig.values()) == {8}
    spec = ok_spec(SET, W=2, nbs=1, nstreams=1, R=1)
    sig = oracle.protocol.expected_final_signals(spec)
    assert len(sig) == 4 and set(sig.values()) == {1}
    cred = oracle.protocol.expected_final_credits(ok_spec(ADD, nbs=5, R=2))
    assert sorted(set(cred.values())) == [2, 3]


@pytest.mark.parametrize("protocol", [ADD, SET])
def test_negative_skip_reset(protocol):
    out = run_random(ok_spec(protocol, skip_reset=True), seed=0)
    assert out.violations, "stale signals must let a consumer read unwritten data"


@pytest.mark.parametrize("protocol", [ADD, SET])
def test_negative_signal_before_fence(protocol):
    _, violations, _ = explore_all(ok_spec(protocol, nbs=1, signal_before_fence=True))
    assert any("read block" in v for v in violations)


@pytest.mark.parametrize("protocol", [ADD, SET])
def test_negative_skip_credit_wait(protocol):
    _, violations, _ = explore_all(ok_spec(protocol, nbs=2, R=1, skip_credit_wait=True))
    assert any("overwrite" in v or "read block" in v for v in violations)


@pytest.mark.parametrize("protocol", [ADD, SET])
def test_negative_missing_piece_times_out(protocol):
    out = run_random(ok_spec(protocol, drop_piece=(1, 0, 1, 0)), seed=3)
    assert not out.completed


def test_signal_ops_and_predicates():
    assert oracle.signal_apply(5, 1, "set") == 1
    assert oracle.signal_apply(5, 3, "add") == 8
    assert oracle.signal_apply(2**64 - 1, 1, "add") == 0
    table = {"eq": (False, True, False), "ne": (True, False, True), "gt": (False, False, True),
             "ge": (False, True, True), "lt": (True, False, False), "le": (True, True, False)}
    for op, want in table.items():
        assert tuple(oracle.compare(v, 4, op) for v in (3, 4, 5)) == want


def test_symm_at():
    base, stride, world = 1 << 40, 1 << 21, 4
    p = base + 1234
    assert oracle.symm_at(base, stride, world, p, 0) == p
    assert oracle.symm_at(base, stride, world, p, 3) == p + 3 * stride
    q = oracle.symm_at(base, stride, world, p, 2)
    assert oracle.symm_at(base, stride, world, q, 1) == p + stride
    assert oracle.symm_at(base, stride, world, q, 2) == q
    assert oracle.symm_at(base, stride, world, p, 4) is None
    assert oracle.symm_at(base, stride, world, p, -1) is None
    assert oracle.symm_at(base, stride, world, base + world * stride, 0) is None
    assert oracle.symm_at(base, stride, world, base - 1, 0) is None


# ---- row units ---------------------------------------------------------------
from oracle.protocol import (RowSpec, explore_rows, expected_final_block_counts,  # noqa: E402
                             expected_row_finals, row_unit_counts, row_units, run_rows_random)


def test_row_unit_counts_worked():
    # S = 37 in S-blocks of 16: rows 16, 16, 5; units of 5 tokens: 4, 4, 1
    assert row_unit_counts(37, 16, 5) == [4, 4, 1]
    # units as large as the block: one each; units of one token: the block's rows
    assert row_unit_counts(37, 16, 16) == [1, 1, 1]
    assert row_unit_counts(37, 16, 1) == [16, 16, 5]
    # the bench workload: 512 tokens in blocks of 64, 8-token units
    assert row_unit_counts(512, 64, 8) == [8] * 8
    assert expected_final_block_counts(37, 16, 5) == [4, 4, 1]


def test_row_unit_counts_brute_force():
    """Each block's unit count equals the number of distinct (block, unit) pairs
    met when every token is assigned to unit (token mod BS) div KU of its block."""
    for S in range(1, 40):
        for BS in range(1, 12):
            for KU in range(1, BS + 1):
                seen = {}
                for s in range(S):
                    seen.setdefault(s // BS, set()).add((s % BS) // KU)
                assert row_unit_counts(S, BS, KU) == [len(seen[b]) for b in sorted(seen)]


def row_spec(protocol, **kw):
    base = dict(W=2, units=(2, 1), nstreams=1, protocol=protocol, n_workers=2, n_consumers=1)
    base.update(kw)
    return RowSpec(**base)


@pytest.mark.parametrize("workers", [2, 3])
@pytest.mark.parametrize("protocol", [ADD, SET])
def test_rows_exhaustive_no_violation(protocol, workers):
    states, violations, stuck = explore_rows(row_spec(protocol, n_workers=workers))
    assert states > 100
    assert violations == [] and not stuck


@pytest.mark.parametrize("protocol", [ADD, SET])
def test_rows_seeded_schedules_match_closed_forms(protocol):
    spec = row_spec(protocol, W=3, units=(3, 3, 1), nstreams=2, n_workers=4, n_consumers=3)
    want_sig, want_cnt = expected_row_finals(spec)
    for seed in range(200):
        out = run_rows_random(spec, seed)
        assert out.completed and out.violations == []
        assert out.signals == want_sig and out.counters == want_cnt
    # every unit is scheduled once
    assert len(row_units(spec)) == 3 * 7


@pytest.mark.parametrize("control", ["skip_reset", "count_before_fence", "signal_every_unit"])
@pytest.mark.parametrize("protocol", [ADD, SET])
def test_rows_negative_controls_fire(control, protocol):
    # three workers: the two units of block 0 of each destination run on different ones
    spec = row_spec(protocol, n_workers=3, **{control: True})
    _, violations, _ = explore_rows(spec)
    assert violations, f"{control} must let a consumer read unpublished rows"


@pytest.mark.parametrize("workers", [2, 3])
@pytest.mark.parametrize("units", [(2, 1), (1, 2), (2, 2)])
def test_rows_share_exhaustive_no_violation(units, workers):
    """ADD shares (each unit of a block with n | W units adds W / n): no consumer
    reads unpublished rows in any interleaving, and the finals are the closed
    forms."""
    spec = row_spec(ADD, units=units, n_workers=workers, share=True)
    states, violations, stuck = explore_rows(spec)
    assert states > 100
    assert violations == [] and not stuck


def test_rows_share_seeded_schedules_match_closed_forms():
    # W = 4: blocks of 4 and 2 units share (4 / 4 = 1, 4 / 2 = 2), 3 units count
    spec = row_spec(ADD, W=4, units=(4, 2, 3, 1), nstreams=2, n_workers=5, n_consumers=3,
                    share=True)
    want_sig, want_cnt = expected_row_finals(spec)
    for seed in range(100):
        out = run_rows_random(spec, seed)
        assert out.completed and out.violations == []
        assert out.signals == want_sig and out.counters == want_cnt


@pytest.mark.parametrize("control", ["share_full", "share_before_fence"])
def test_rows_share_negative_controls_fire(control):
    spec = row_spec(ADD, units=(2, 1), n_workers=3, share=True, **{control: True})
    _, violations, _ = explore_rows(spec)
    assert violations, f"{control} must let a consumer read unpublished rows"


def test_piece_counts_worked():
    from oracle.protocol import expected_final_piece_counts
    # the MoE-combine shape: 32-token tiles cut into 8-token pieces, 8 sources, ADD
    assert expected_final_piece_counts(4096, 32, 8, 8, ADD) == [32] * 128
    # ragged: S = 37, tiles of 16, pieces of 6 -> parts 3, 3, 1; SET counts per source
    assert expected_final_piece_counts(37, 16, 6, 3, SET) == [3, 3, 1]
    assert expected_final_piece_counts(37, 16, 6, 3, ADD) == [9, 9, 3]
