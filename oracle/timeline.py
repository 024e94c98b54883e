"""Discrete-event model of a copy -> compute software pipeline.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Source: TileLang tutorial, chapter 11 "pipeline and autotuning":
  * section 1.2 -- three quantities in cycles: the cost of issuing a copy
    (``issue``), the time from issue until the data has arrived (``latency``),
    and the time one iteration's compute takes (``compute``); issue and arrival
    are separate events on modern accelerators.
  * section 1.3 -- a greedy list schedule over (issue, latency, compute,
    stages) that yields every iteration's copy and compute times; its summary
    table for 8 iterations, issue=1, latency=30, compute=20 is the worked
    example this model must reproduce; the minimum sufficient depth is
    1 + ceil(latency / compute).
  * section 1.4 -- the same model at 16 iterations.
  * section 2.2 -- the steady-state period max(compute, issue,
    (latency + compute) / depth), i.e. each buffer is held from the moment its
    copy is issued until its compute has finished.
  * section 2.3 / 5.2 -- with ``stages`` buffers, iteration i uses slot
    i mod stages; a slot may be written again only after the compute that
    read it has finished.

The page prints the model's output but not its code.  The reading taken here
(every rule below is one of the statements above):
  * copies are issued in order on one issue lane, ``issue`` cycles apart;
  * copy i may not be issued before the compute of iteration i - stages has
    ended (its slot is still being read until then);
  * the data of copy i is ready ``latency`` cycles after its issue;
  * computes run in order on one compute lane; compute i starts when its data
    is ready and compute i-1 has ended, and lasts ``compute`` cycles.
With stages = 1 the copy of iteration i waits for compute i-1, so every round
costs latency + compute -- the non-pipelined loop of section 1.1.

Summary quantities, as named in the printed table:
  makespan      end of the last compute
  speedup       makespan(stages=1) / makespan(stages)
  issue_iv      mean interval between consecutive copy issues
  compute_iv    mean interval between consecutive compute starts
  compute_util  busy compute cycles / (makespan - first compute start)
"""
from dataclasses import dataclass, field
from math import ceil
from typing import List


@dataclass
class Schedule:
    iterations: int
    issue: float
    latency: float
    compute: float
    stages: int
    issue_start: List[float] = field(default_factory=list)
    ready: List[float] = field(default_factory=list)
    compute_start: List[float] = field(default_factory=list)
    compute_end: List[float] = field(default_factory=list)

    @property
    def makespan(self) -> float:
        return self.compute_end[-1] if self.compute_end else 0.0

    @property
    def issue_iv(self) -> float:
        n = self.iterations
        return (self.issue_start[-1] - self.issue_start[0]) / (n - 1) if n > 1 else 0.0

    @property
    def compute_iv(self) -> float:
        n = self.iterations
        return (self.compute_start[-1] - self.compute_start[0]) / (n - 1) if n > 1 else 0.0

    @property
    def compute_util(self) -> float:
        busy = self.iterations * self.compute
        span = self.makespan - self.compute_start[0]
        return busy / span if span > 0 else 1.0


def simulate(iterations: int, issue: float, latency: float, compute: float, stages: int) -> Schedule:
    """Greedy schedule of `iterations` copy->compute rounds over `stages` buffers."""
    if iterations < 1 or stages < 1:
        raise ValueError("iterations and stages must be >= 1")
    if issue < 0 or latency < 0 or compute < 0:
        raise ValueError("cycle counts must be non-negative")
    s = Schedule(iterations, issue, latency, compute, stages)
    for i in range(iterations):
        t_issue = s.issue_start[i - 1] + issue if i > 0 else 0.0
        if i >= stages:  # slot i mod stages is free once compute i - stages ends
            t_issue = max(t_issue, s.compute_end[i - stages])
        t_ready = t_issue + latency
        t_start = max(t_ready, s.compute_end[i - 1]) if i > 0 else t_ready
        s.issue_start.append(t_issue)
        s.ready.append(t_ready)
        s.compute_start.append(t_start)
        s.compute_end.append(t_start + compute)
    return s


def speedup(iterations: int, issue: float, latency: float, compute: float, stages: int) -> float:
    """makespan at one buffer divided by makespan at `stages` buffers."""
    base = simulate(iterations, issue, latency, compute, 1).makespan
    return base / simulate(iterations, issue, latency, compute, stages).makespan


def min_depth(latency: float, compute: float) -> int:
    """Smallest buffer count that reaches the compute-bound steady state.

    The producer has to run ceil(latency / compute) iterations ahead of the
    consumer to cover one copy's flight time, plus the buffer being read.
    """
    if compute <= 0:
        raise ValueError("compute must be positive")
    return 1 + int(ceil(latency / compute))


def steady_period(issue: float, latency: float, compute: float, stages: int) -> float:
    """Closed-form cycles per iteration once the pipeline is full.

    A buffer is occupied from its copy's issue until its compute ends, at least
    latency + compute cycles, so `stages` buffers admit at most `stages` rounds
    per (latency + compute); the compute lane and the issue lane bound the
    period from below as well.
    """
    return max(compute, issue, (latency + compute) / stages)


def summary_rows(iterations: int, issue: float, latency: float, compute: float, stages_list):
    """The per-depth summary the model prints: one dict per stage count."""
    base = simulate(iterations, issue, latency, compute, 1).makespan
    rows = []
    for st in stages_list:
        s = simulate(iterations, issue, latency, compute, st)
        rows.append(dict(stages=st, makespan=s.makespan, speedup=base / s.makespan,
                         issue_iv=s.issue_iv, compute_iv=s.compute_iv, compute_util=s.compute_util))
    return rows

