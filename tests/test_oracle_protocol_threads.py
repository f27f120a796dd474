"""The signal protocol run by real host threads (oracle/protocol_threads.c).

Second executor of the protocol model: one producer thread per source and one
consumer thread per destination on C11 release/acquire atomics, with seeded
random delays, checked by ThreadSanitizer and by the closed forms (the combine's
output map, final signals W under ADD and 1 under SET, credits equal to each ring
slot's uses).  The negative controls must each be caught: a signal issued before
the data (a race), signals not zeroed before the launch (a race and wrong final
state), a piece never sent (a bounded wait that times out).
"""
import os
import shutil
import subprocess

import pytest

from oracle import build as oracle_build

SRC = oracle_build.THREADS_SRC
TSAN_REPORT = "WARNING: ThreadSanitizer"


@pytest.fixture(scope="module")
def tsan_exe(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not installed")
    exe = str(tmp_path_factory.mktemp("tsan") / "protocol_threads_tsan")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-Wall", "-Wextra", "-fsanitize=thread", SRC, "-o", exe, "-lpthread"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("ThreadSanitizer build unavailable: " + r.stderr[-300:])
    return exe


@pytest.fixture(scope="module")
def plain_exe():
    oracle_build.build()
    return oracle_build.THREADS_EXE


def run(exe, W, S, B, X, R, op, seed, control=None, wait_s=None):
    args = [exe, str(W), str(S), str(B), str(X), str(R), op, str(seed)] + ([control] if control else [])
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=0")
    if wait_s is not None:
        env["PROTOCOL_WAIT_S"] = str(wait_s)
    r = subprocess.run(args, capture_output=True, text=True, timeout=120, env=env)
    return r.returncode, r.stdout.strip(), r.stderr


CASES = [
    # W, S, B (rows per tile), X (elements per row), R (ring slots; 0 = a slot per tile), op
    (1, 4, 1, 3, 1, "add"),
    (2, 8, 2, 4, 0, "set"),
    (2, 8, 1, 4, 1, "add"),    # a one-slot ring: every tile waits for the previous hand-back
    (3, 12, 3, 5, 2, "set"),
    (4, 16, 2, 8, 0, "add"),
    (4, 16, 2, 8, 2, "add"),
    (4, 16, 4, 8, 3, "set"),   # T = 4 tiles on a 3-slot ring: slots used 2, 1, 1 times
    (8, 32, 4, 16, 3, "add"),
    (8, 32, 4, 16, 1, "set"),
]


@pytest.mark.parametrize("W,S,B,X,R,op", CASES)
def test_clean_runs_race_free_and_exact(tsan_exe, W, S, B, X, R, op):
    for seed in range(3):
        rc, out, err = run(tsan_exe, W, S, B, X, R, op, seed)
        assert TSAN_REPORT not in err, err[-2000:]
        assert (rc, out) == (0, "ok"), (rc, out, err[-500:])


@pytest.mark.parametrize("W,S,B,X,R,op", CASES)
def test_many_seeds_uninstrumented(plain_exe, W, S, B, X, R, op):
    for seed in range(20):
        assert run(plain_exe, W, S, B, X, R, op, seed)[:2] == (0, "ok"), seed


@pytest.mark.parametrize("R,op", [(0, "add"), (2, "add"), (0, "set"), (2, "set")])
def test_signal_before_data_is_a_race(tsan_exe, R, op):
    rc, out, err = run(tsan_exe, 4, 16, 2, 8, R, op, 1, "--signal-first")
    assert TSAN_REPORT in err and "data race" in err, (rc, out)


@pytest.mark.parametrize("R,op", [(0, "add"), (2, "add"), (0, "set"), (2, "set")])
def test_skipped_reset_is_caught(tsan_exe, R, op):
    rc, out, err = run(tsan_exe, 4, 16, 2, 8, R, op, 1, "--no-reset")
    assert rc != 0
    assert TSAN_REPORT in err or out.startswith("mismatch"), (rc, out)
    if op == "add":
        assert out.startswith("mismatch")  # W extra ADDs leave every tile signal at 2 W


@pytest.mark.parametrize("R,op", [(0, "add"), (2, "set")])
def test_missing_piece_times_out(plain_exe, R, op):
    rc, out, _ = run(plain_exe, 4, 16, 2, 8, R, op, 1, "--drop-piece", wait_s=0.5)
    assert (rc, out) == (2, "timeout")


def test_bad_arguments_rejected(plain_exe):
    assert run(plain_exe, 4, 15, 2, 8, 0, "add", 0)[0] == 3   # S not a multiple of B
    assert run(plain_exe, 4, 16, 2, 8, 0, "xor", 0)[0] == 3
