"""Model of the tile-signalled producer/consumer protocol -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
this module; the GPU path never imports it.

What it models (the Reverse All2All page, "Reverse All2All (EP MoE Distributed
Kernel)": "MTE Implementation > Signal-Based Synchronization" and "Wait/Notify
Optimization > Dual Signal Memory Region Design"; the HyperParallel RFC, section
5.1 "Push 模式" and section 六 ``shmem_put_with_signal``):

* a producer piece (source r -> destination j, stream t, S-block b):
    1. wait until the ring slot b mod R of (j, t) has been handed back for the
       previous use (credit count >= b div R), acquire;
    2. write its data into destination j's staging slot;
    3. fence: the data is published before the signal;
    4. signal on destination j: SET 1 on the piece's own slot (one signal per
       (src, dst) piece) or ADD 1 on the tile's slot (push mode, the consumer
       waits for W).
* a consumer unit on destination j (the whole tile (j, t, b) under ADD, one
  piece (j, t, b, r) under SET):
    1. wait until the signal equals its expected value (W under ADD, 1 under
       SET), acquire; the wait does not consume the signal;
    2. read the staging slot(s);
    3. fence, then hand the ring slot back: the slot's credit count grows by 1.

Readings taken where the pages leave a step open:
* credits are counts of completed consumptions (monotone), not a flag reset to
  0 by the consumer; the producer of use u of a slot waits for count >= u.  The
  pages' "wait for 0, notify 1, consumer notifies 0" handshake is the same
  hand-off for one piece per slot; a count also works when W producers share
  one tile and never needs a reset inside a launch;
* tile signals are unique per (destination, S-block, stream) and are never
  reset inside a launch (the dual-region design's "write once use once" data
  signals); the host zeroes both regions before every launch.

Memory is modelled weakly enough to catch the protocol's classic bugs: a write
is "pending" (invisible to readers) until its producer's fence publishes it.
A reader that finds anything but the block it expects records a violation; so
does a writer that overwrites a slot whose previous block was never consumed.
"""
from __future__ import annotations

import dataclasses
import random
from typing import Dict, List, Optional, Tuple

SET = "set"
ADD = "add"


@dataclasses.dataclass(frozen=True)
class ProtocolSpec:
    W: int              # simulated ranks
    nbs: int            # S-blocks per stream
    nstreams: int       # streams per destination (head blocks x D blocks)
    R: int              # ring depth, in S-blocks
    protocol: str       # SET | ADD
    n_producers: int = 2
    n_consumers: int = 2
    # negative controls (each turns one rule of the protocol off)
    skip_reset: bool = False          # signals keep the previous launch's final values
    signal_before_fence: bool = False  # signal published before the data
    skip_credit_wait: bool = False     # producer ignores the ring hand-back
    drop_piece: Optional[Tuple[int, int, int, int]] = None  # (j, t, b, r) never produced


def pieces(spec: ProtocolSpec) -> List[Tuple[int, int, int, int]]:
    """All producer pieces (j, t, b, r), S-block major."""
    return [(j, t, b, r) for b in range(spec.nbs) for j in range(spec.W)
            for t in range(spec.nstreams) for r in range(spec.W)]


def units(spec: ProtocolSpec) -> List[tuple]:
    """All consumer units: (j, t, b) under ADD, (j, t, b, r) under SET; S-block major."""
    if spec.protocol == ADD:
        return [(j, t, b) for b in range(spec.nbs) for j in range(spec.W)
                for t in range(spec.nstreams)]
    return [(j, t, b, r) for b in range(spec.nbs) for j in range(spec.W)
            for t in range(spec.nstreams) for r in range(spec.W)]


def signal_key(spec: ProtocolSpec, j, t, b, r):
    return (j, t, b) if spec.protocol == ADD else (j, t, b, r)


def credit_key(spec: ProtocolSpec, j, t, b, r):
    slot = b % spec.R
    return (j, t, slot) if spec.protocol == ADD else (j, t, slot, r)


def expected_final_signals(spec: ProtocolSpec) -> Dict[tuple, int]:
    """Closed-form final tile signals: every ADD tile holds W, every SET piece holds 1."""
    val = spec.W if spec.protocol == ADD else 1
    keys = {signal_key(spec, j, t, b, r) for (j, t, b, r) in pieces(spec)}
    return {k: val for k in keys}


def expected_final_credits(spec: ProtocolSpec) -> Dict[tuple, int]:
    """Closed-form final credit counts: the number of S-blocks that used each ring slot."""
    out: Dict[tuple, int] = {}
    for (j, t, b, r) in pieces(spec):
        k = credit_key(spec, j, t, b, r)
        if k not in out:
            out[k] = 0
    for k in out:
        slot = k[2]
        out[k] = len(range(slot, spec.nbs, spec.R))
    return out


class _Run:
    """One execution of the protocol; agents advance one step at a time."""

    def __init__(self, spec: ProtocolSpec):
        self.spec = spec
        ps = [p for p in pieces(spec) if p != spec.drop_piece]
        us = units(spec)
        self.prod_lists = [ps[i::spec.n_producers] for i in range(spec.n_producers)]
        self.cons_lists = [us[i::spec.n_consumers] for i in range(spec.n_consumers)]
        # (list index, step) per agent
        self.prod_pc = [[0, 0] for _ in self.prod_lists]
        self.cons_pc = [[0, 0] for _ in self.cons_lists]
        self.sig: Dict[tuple, int] = {}
        if spec.skip_reset:
            self.sig = dict(expected_final_signals(spec))
        self.credit: Dict[tuple, int] = {}
        self.visible: Dict[tuple, int] = {}    # staging (j, t, slot, r) -> block held
        self.pending: Dict[tuple, int] = {}
        self.consumed: Dict[tuple, bool] = {}  # (j, t, b, r) consumed?
        self.out: Dict[tuple, Optional[int]] = {}  # (j, t, b, r) -> block read
        self.violations: List[str] = []

    # ---- producer --------------------------------------------------------
    def _prod_steps(self):
        if self.spec.signal_before_fence:
            return ("wait", "write", "signal", "fence")
        return ("wait", "write", "fence", "signal")

    def prod_runnable(self, a: int) -> bool:
        li, st = self.prod_pc[a]
        lst = self.prod_lists[a]
        if li >= len(lst):
            return False
        if self._prod_steps()[st] != "wait" or self.spec.skip_credit_wait:
            return True
        j, t, b, r = lst[li]
        return self.credit.get(credit_key(self.spec, j, t, b, r), 0) >= b // self.spec.R

    def prod_step(self, a: int) -> None:
        li, st = self.prod_pc[a]
        j, t, b, r = self.prod_lists[a][li]
        slot = (j, t, b % self.spec.R, r)
        kind = self._prod_steps()[st]
        if kind == "write":
            old = self.visible.get(slot)
            if old is not None and not self.consumed.get((j, t, old, r), False):
                self.violations.append(f"overwrite of unconsumed block {old} at {slot}")
            self.pending[slot] = b
        elif kind == "fence":
            if slot in self.pending:
                self.visible[slot] = self.pending.pop(slot)
        elif kind == "signal":
            k = signal_key(self.spec, j, t, b, r)
            if self.spec.protocol == ADD:
                self.sig[k] = self.sig.get(k, 0) + 1
            else:
                self.sig[k] = 1
        st += 1
        if st == 4:
            li, st = li + 1, 0
        self.prod_pc[a] = [li, st]

    # ---- consumer --------------------------------------------------------
    def cons_runnable(self, a: int) -> bool:
        li, st = self.cons_pc[a]
        lst = self.cons_lists[a]
        if li >= len(lst):
            return False
        if st != 0:
            return True
        u = lst[li]
        want = self.spec.W if self.spec.protocol == ADD else 1
        return self.sig.get(u, 0) == want

    def cons_step(self, a: int) -> None:
        li, st = self.cons_pc[a]
        u = self.cons_lists[a][li]
        if self.spec.protocol == ADD:
            j, t, b = u
            rs = range(self.spec.W)
        else:
            j, t, b, r0 = u
            rs = (r0,)
        if st == 1:  # read
            for r in rs:
                got = self.visible.get((j, t, b % self.spec.R, r))
                self.out[(j, t, b, r)] = got
                if got != b:
                    self.violations.append(f"unit {u} read block {got} from source {r}, "
                                           f"expected {b}")
                self.consumed[(j, t, b, r)] = True
        elif st == 2:  # fence + credit hand-back
            k = credit_key(self.spec, j, t, b, rs[0])
            self.credit[k] = self.credit.get(k, 0) + 1
        st += 1
        if st == 3:
            li, st = li + 1, 0
        self.cons_pc[a] = [li, st]

    # ---- whole system ----------------------------------------------------
    def agents(self):
        return ([("p", a) for a in range(len(self.prod_lists))]
                + [("c", a) for a in range(len(self.cons_lists))])

    def runnable(self):
        out = []
        for kind, a in self.agents():
            if (self.prod_runnable(a) if kind == "p" else self.cons_runnable(a)):
                out.append((kind, a))
        return out

    def step(self, agent) -> None:
        kind, a = agent
        if kind == "p":
            self.prod_step(a)
        else:
            self.cons_step(a)

    def done(self) -> bool:
        return (all(pc[0] >= len(l) for pc, l in zip(self.prod_pc, self.prod_lists))
                and all(pc[0] >= len(l) for pc, l in zip(self.cons_pc, self.cons_lists)))

    def key(self):
        return (tuple(map(tuple, self.prod_pc)), tuple(map(tuple, self.cons_pc)),
                tuple(sorted(self.sig.items())), tuple(sorted(self.credit.items())),
                tuple(sorted(self.visible.items())), tuple(sorted(self.pending.items())),
                tuple(sorted(self.consumed.items())), bool(self.violations))

    def clone(self) -> "_Run":
        c = _Run.__new__(_Run)
        c.spec = self.spec
        c.prod_lists = self.prod_lists
        c.cons_lists = self.cons_lists
        c.prod_pc = [list(x) for x in self.prod_pc]
        c.cons_pc = [list(x) for x in self.cons_pc]
        c.sig = dict(self.sig)
        c.credit = dict(self.credit)
        c.visible = dict(self.visible)
        c.pending = dict(self.pending)
        c.consumed = dict(self.consumed)
        c.out = dict(self.out)
        c.violations = list(self.violations)
        return c


@dataclasses.dataclass
class Outcome:
    completed: bool           # every agent finished (no deadlock / time-out)
    violations: List[str]
    signals: Dict[tuple, int]
    credits: Dict[tuple, int]
    out: Dict[tuple, Optional[int]]


def run_random(spec: ProtocolSpec, seed: int, max_steps: int = 1_000_000) -> Outcome:
    """One execution under a seeded random scheduler."""
    rng = random.Random(seed)
    run = _Run(spec)
    for _ in range(max_steps):
        if run.done():
            break
        ready = run.runnable()
        if not ready:
            break  # every remaining agent spins forever: the bounded wait times out
        run.step(rng.choice(ready))
    return Outcome(run.done(), run.violations, run.sig, run.credit, run.out)


def explore_all(spec: ProtocolSpec, max_states: int = 2_000_000) -> Tuple[int, List[str], bool]:
    """Every interleaving (depth-first over distinct states).

    Returns (states visited, violations found on any path, some path deadlocked).
    """
    seen = set()
    stack = [_Run(spec)]
    violations: List[str] = []
    deadlock = False
    while stack:
        run = stack.pop()
        k = run.key()
        if k in seen:
            continue
        seen.add(k)
        if len(seen) > max_states:
            raise RuntimeError("state space too large for exhaustive exploration")
        if run.violations:
            violations.extend(run.violations)
            continue
        if run.done():
            continue
        ready = run.runnable()
        if not ready:
            deadlock = True
            continue
        for ag in ready:
            nxt = run.clone()
            nxt.step(ag)
            stack.append(nxt)
    return len(seen), violations, deadlock


# ---------------------------------------------------------------------------
# Row units: the combine's work cut into units that each fill whole output
# rows with every source's data, completed per S-block by an arrival count.
#
# This is the push mode of the HyperParallel RFC (section 5.1) with one work
# unit carrying all W sources of some token rows instead of one source's piece
# of a tile.  The tile signal keeps the pages' meaning -- the tile is complete
# once it reads W (ADD) or each of its (tile, source) slots reads 1 (SET) -- and
# a block counter decides which unit may give it that value:
#   * a unit writes its rows (all sources) into out_j, fences (publishes them),
#     then adds 1 to the arrival counter of its S-block (j, b);
#   * the unit whose add brings the counter to the block's unit count signals
#     every tile of the block: ADD W on each tile slot, or SET 1 on each (tile,
#     source) slot -- the values W per-source pieces would have left.
# Variant (share): under ADD, in a block whose unit count n divides W, every
# unit adds W / n to each tile of its block after its own fence, and still
# counts itself; a tile then reads W exactly when all n units have published
# their rows, with no unit waiting for the count.
# Readings where the pages say nothing (they have no row units): the counter is
# a monotone count of arrivals zeroed with the signals before the launch, and
# it ends at the block's unit count.  Visibility is modelled as above (a write
# is pending until its writer's fence), so the model checks the counting logic;
# the device-wide acquire/release pair the completing unit runs on the GPU is
# what makes the other units' fences cumulative there.


def row_unit_counts(S: int, BS: int, KU: int) -> List[int]:
    """Units of each S-block: ceil(rows of the block / tokens per unit)."""
    out = []
    for b in range(-(-S // BS)):
        rows = min(BS, S - b * BS)
        out.append(-(-rows // KU))
    return out


def expected_final_block_counts(S: int, BS: int, KU: int) -> List[int]:
    """Closed-form final arrival counters: each block's counter ends at its unit count."""
    return row_unit_counts(S, BS, KU)


@dataclasses.dataclass(frozen=True)
class RowSpec:
    W: int
    units: Tuple[int, ...]   # unit count of each S-block
    nstreams: int            # signal tiles per (destination, S-block)
    protocol: str            # SET | ADD
    n_workers: int = 2       # units are dealt round-robin, as the static schedule does
    n_consumers: int = 2
    # negative controls
    skip_reset: bool = False          # counters and signals keep the previous launch's finals
    count_before_fence: bool = False  # the arrival is counted before the rows are published
    signal_every_unit: bool = False   # no counter: each unit signals its block on its own
    share: bool = False               # ADD, n | W: each unit adds W / n after its fence
    share_full: bool = False          # negative control: each sharing unit adds all of W
    share_before_fence: bool = False  # negative control: the share is added before the fence


def row_units(spec: RowSpec) -> List[Tuple[int, int, int]]:
    """All units (j, b, k), in the static schedule's order: block, unit, destination."""
    return [(j, b, k) for b, n in enumerate(spec.units) for k in range(n) for j in range(spec.W)]


def expected_row_finals(spec: RowSpec) -> Tuple[Dict[tuple, int], Dict[tuple, int]]:
    """(tile signals, block counters) after a launch, in closed form."""
    ps = ProtocolSpec(W=spec.W, nbs=len(spec.units), nstreams=spec.nstreams, R=1,
                      protocol=spec.protocol)
    cnt = {(j, b): n for j in range(spec.W) for b, n in enumerate(spec.units)}
    return expected_final_signals(ps), cnt


class _RowRun:
    def __init__(self, spec: RowSpec):
        self.spec = spec
        us = row_units(spec)
        self.work = [us[i::spec.n_workers] for i in range(spec.n_workers)]
        cons = []
        for b in range(len(spec.units)):
            for j in range(spec.W):
                for t in range(spec.nstreams):
                    if spec.protocol == ADD:
                        cons.append((j, t, b))
                    else:
                        cons.extend((j, t, b, r) for r in range(spec.W))
        self.cons = [cons[i::spec.n_consumers] for i in range(spec.n_consumers)]
        self.wpc = [[0, 0] for _ in self.work]
        self.cpc = [[0, 0] for _ in self.cons]
        sig0, cnt0 = expected_row_finals(spec) if spec.skip_reset else ({}, {})
        self.sig: Dict[tuple, int] = dict(sig0)
        self.cnt: Dict[tuple, int] = dict(cnt0)
        self.last: Dict[tuple, bool] = {}
        self.pending = set()   # (j, b, k) rows written, not yet published
        self.visible = set()
        self.violations: List[str] = []

    def _shares(self, b):
        """Whether the units of block b add shares (ADD, unit count divides W)."""
        return self.spec.share and self.spec.protocol == ADD and self.spec.W % self.spec.units[b] == 0

    def _steps(self, b=0):
        if self.spec.signal_every_unit:
            return ("write", "fence", "signal")
        if self._shares(b) and self.spec.share_before_fence:
            return ("write", "signal", "fence", "count")
        if self.spec.count_before_fence:
            return ("write", "count", "fence", "signal")
        return ("write", "fence", "count", "signal")

    def _signal_block(self, j, b, amount=None):
        for t in range(self.spec.nstreams):
            if self.spec.protocol == ADD:
                self.sig[(j, t, b)] = self.sig.get((j, t, b), 0) + (self.spec.W if amount is None else amount)
            else:
                for r in range(self.spec.W):
                    self.sig[(j, t, b, r)] = 1

    def work_runnable(self, a):
        return self.wpc[a][0] < len(self.work[a])

    def work_step(self, a):
        li, st = self.wpc[a]
        u = self.work[a][li]
        j, b, k = u
        steps = self._steps(b)
        kind = steps[st]
        if kind == "write":
            self.pending.add(u)
        elif kind == "fence":
            if u in self.pending:
                self.pending.discard(u)
                self.visible.add(u)
        elif kind == "count":
            c = self.cnt.get((j, b), 0) + 1
            self.cnt[(j, b)] = c
            self.last[u] = c == self.spec.units[b]
        elif kind == "signal":
            if self._shares(b):
                n = self.spec.units[b]
                self._signal_block(j, b, self.spec.W if self.spec.share_full else self.spec.W // n)
            elif self.spec.signal_every_unit or self.last.get(u, False):
                self._signal_block(j, b)
        st += 1
        if st == len(steps):
            li, st = li + 1, 0
        self.wpc[a] = [li, st]

    def cons_runnable(self, a):
        li, st = self.cpc[a]
        if li >= len(self.cons[a]):
            return False
        if st:
            return True
        c = self.cons[a][li]
        want = self.spec.W if self.spec.protocol == ADD else 1
        return self.sig.get(c, 0) == want

    def cons_step(self, a):
        li, st = self.cpc[a]
        c = self.cons[a][li]
        j, b = c[0], c[2]
        for k in range(self.spec.units[b]):
            if (j, b, k) not in self.visible:
                self.violations.append(f"consumer {c} read unpublished rows of unit {(j, b, k)}")
        self.cpc[a] = [li + 1, 0]

    def agents(self):
        return [("w", a) for a in range(len(self.work))] + [("c", a) for a in range(len(self.cons))]

    def runnable(self):
        return [(k, a) for k, a in self.agents()
                if (self.work_runnable(a) if k == "w" else self.cons_runnable(a))]

    def step(self, ag):
        k, a = ag
        if k == "w":
            self.work_step(a)
        else:
            self.cons_step(a)

    def done(self):
        return (all(pc[0] >= len(l) for pc, l in zip(self.wpc, self.work))
                and all(pc[0] >= len(l) for pc, l in zip(self.cpc, self.cons)))

    def key(self):
        return (tuple(map(tuple, self.wpc)), tuple(map(tuple, self.cpc)),
                tuple(sorted(self.sig.items())), tuple(sorted(self.cnt.items())),
                tuple(sorted(self.last.items())), tuple(sorted(self.pending)),
                tuple(sorted(self.visible)), bool(self.violations))

    def clone(self):
        c = _RowRun.__new__(_RowRun)
        c.spec, c.work, c.cons = self.spec, self.work, self.cons
        c.wpc = [list(x) for x in self.wpc]
        c.cpc = [list(x) for x in self.cpc]
        c.sig, c.cnt, c.last = dict(self.sig), dict(self.cnt), dict(self.last)
        c.pending, c.visible = set(self.pending), set(self.visible)
        c.violations = list(self.violations)
        return c


@dataclasses.dataclass
class RowOutcome:
    completed: bool
    violations: List[str]
    signals: Dict[tuple, int]
    counters: Dict[tuple, int]


def run_rows_random(spec: RowSpec, seed: int, max_steps: int = 1_000_000) -> RowOutcome:
    """One execution of the row-unit protocol under a seeded random scheduler."""
    rng = random.Random(seed)
    run = _RowRun(spec)
    for _ in range(max_steps):
        if run.done():
            break
        ready = run.runnable()
        if not ready:
            break  # the remaining consumers spin until their bounded wait gives up
        run.step(rng.choice(ready))
    return RowOutcome(run.done(), run.violations, run.sig, run.cnt)


def explore_rows(spec: RowSpec, max_states: int = 2_000_000) -> Tuple[int, List[str], bool]:
    """Every interleaving of the row-unit protocol: (states, violations, some path stuck)."""
    seen = set()
    stack = [_RowRun(spec)]
    violations: List[str] = []
    stuck = False
    while stack:
        run = stack.pop()
        k = run.key()
        if k in seen:
            continue
        seen.add(k)
        if len(seen) > max_states:
            raise RuntimeError("state space too large for exhaustive exploration")
        if run.violations:
            violations.extend(run.violations)
            continue
        if run.done():
            continue
        ready = run.runnable()
        if not ready:
            stuck = True
            continue
        for ag in ready:
            nxt = run.clone()
            nxt.step(ag)
            stack.append(nxt)
    return len(seen), violations, stuck


def expected_final_piece_counts(S: int, BS: int, PR: int, W: int, protocol: str) -> List[int]:
    """Direct mode with tiles cut into pieces of PR tokens: the arrival counter of a
    tile ends at the number of pieces that fed it -- ceil(rows of its S-block / PR)
    from each of the W sources under ADD (one counter per tile), from its one source
    under SET (one counter per tile and source).  Per S-block."""
    per_source = row_unit_counts(S, BS, PR)
    return [n * W for n in per_source] if protocol == ADD else per_source
