"""Cross-resource staggering of several request groups on one GPU.

VeriCache summary, "P1 cross-resource staggering": drafting is bound by HBM
bandwidth and verification by the link that brings the full cache from host
memory, so the runtime interleaves requests: while one group verifies (its
full cache crossing the host link), another drafts on the compute units.

Each group is an Engine with its own compute stream and its own copy stream
(full cache in pinned host memory, staged in chunks: "Architecture support",
long-context decoding). The scheduler issues the groups' rounds in turn with
no host synchronisation. The only ordering it adds is on the compute units:
a group's draft steps start once the previous group's draft steps of the
same turn have ended, so drafting alternates between groups, while every
group's copies and verification proceed on their own streams as soon as
their data allow. Optional timing events on every stream give each
resource's busy time: the host link (chunk copies) and drafting.
"""
from __future__ import annotations

import dataclasses

import torch

from .configs import RoundConfig
from .engine import Engine


def merge(intervals) -> list:
    """The disjoint intervals covering the same points as (start, end) pairs."""
    out = []
    for a, b in sorted(intervals):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return [(a, b) for a, b in out]


def union_length(intervals) -> float:
    """Total length covered by a set of (start, end) intervals."""
    return sum(b - a for a, b in merge(intervals))


def intersection_length(xs, ys) -> float:
    """Length covered by both interval sets."""
    total = 0.0
    for a, b in merge(xs):
        for c, d in merge(ys):
            total += max(0.0, min(b, d) - max(a, c))
    return total


@dataclasses.dataclass
class RunStats:
    groups: int
    rounds: int
    wall_s: float
    committed_tokens: int
    link_busy_s: float | None = None
    draft_busy_s: float | None = None
    overlap_s: float | None = None
    link_bytes: int | None = None

    @property
    def tok_s(self) -> float:
        return self.committed_tokens / self.wall_s

    @property
    def group_rounds_s(self) -> float:
        """Rounds of all groups per second: the throughput measure that does
        not depend on how many drafts each group's data lets it accept."""
        return self.groups * self.rounds / self.wall_s

    def as_dict(self) -> dict:
        d = dataclasses.asdict(self)
        d["tok_s"] = self.tok_s
        d["group_rounds_s"] = self.group_rounds_s
        if self.link_busy_s is not None:
            d["link_busy_frac"] = self.link_busy_s / self.wall_s
            d["draft_busy_frac"] = self.draft_busy_s / self.wall_s
            d["overlap_frac"] = self.overlap_s / self.wall_s
            d["link_GBs_while_busy"] = self.link_bytes / self.link_busy_s / 1e9 if self.link_busy_s else 0.0
        return d


class StaggeredGroups:
    """n_groups request groups of one layer shape, each an Engine with a
    host-resident full cache on its own streams (group g draws its inputs
    from seed cfg.seed + 1000 g)."""

    def __init__(self, cfg: RoundConfig, n_groups: int, rounds_cap: int, device: str = "cuda"):
        if not cfg.staged:
            raise ValueError("staggering needs the full cache in host memory (a staged configuration)")
        self.cfg = cfg
        self.groups = [Engine(cfg.scaled(name=f"{cfg.name}-g{g}", seed=cfg.seed + 1000 * g), rounds_cap=rounds_cap,
                              device=device, stream=torch.cuda.Stream(torch.device(device)))
                       for g in range(n_groups)]
        torch.cuda.synchronize(torch.device(device))

    def run(self, rounds: int, trace: bool = False, n_groups: int | None = None) -> RunStats:
        """Issue `rounds` rounds of every group (or of the first n_groups),
        drafting staggered across groups; returns committed tokens and wall
        time (and, with trace, the busy time of the host link and of
        drafting, from events)."""
        import time

        groups = self.groups[:n_groups] if n_groups else self.groups
        dev = groups[0].dev
        k = self.cfg.k
        ev_pairs_draft = []
        start = torch.cuda.Event(enable_timing=True)
        if trace:
            for e in groups:
                e.copy_events = []
        torch.cuda.synchronize(dev)
        first = [e.round_idx for e in groups]
        t0 = time.perf_counter()
        start.record(groups[0].stream)
        for e in groups[1:]:
            e.stream.wait_event(start)
        prev_draft = None
        for _ in range(rounds):
            for e in groups:
                e.begin_round()  # the first chunks of the full cache cross the link from now on
                if prev_draft is not None:
                    e.stream.wait_event(prev_draft)
                if trace:
                    a = torch.cuda.Event(enable_timing=True)
                    a.record(e.stream)
                for j in range(k):
                    e.draft_step(j)
                prev_draft = torch.cuda.Event(enable_timing=trace)
                prev_draft.record(e.stream)
                if trace:
                    ev_pairs_draft.append((a, prev_draft))
                e.embed_block()
                e.verify_attention()
                e.verify_vocab()
                e.accept_commit()
        torch.cuda.synchronize(dev)
        wall = time.perf_counter() - t0
        tokens = int(sum(int((e.n_accept[f:f + rounds] + 1).sum()) for e, f in zip(groups, first)))
        st = RunStats(groups=len(groups), rounds=rounds, wall_s=wall, committed_tokens=tokens)
        if trace:
            copies = [(start.elapsed_time(a) * 1e-3, start.elapsed_time(b) * 1e-3, n)
                      for e in groups for a, b, n in e.copy_events]
            drafts = [(start.elapsed_time(a) * 1e-3, start.elapsed_time(b) * 1e-3) for a, b in ev_pairs_draft]
            cint = [(a, b) for a, b, _ in copies]
            st.link_busy_s = union_length(cint)
            st.draft_busy_s = union_length(drafts)
            st.overlap_s = intersection_length(cint, drafts)
            st.link_bytes = sum(n for _, _, n in copies)
            for e in groups:
                e.copy_events = None
        return st
