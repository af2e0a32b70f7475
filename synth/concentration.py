"""KV-concentration workload simulator: synchronous waves against continuous
refill of B decode slots, with an optional KV page budget.

KV4-RL pages (onedev.kr summary, "어떻게 동작하나"; paper.rainbus.top
summary, "研究动机" and "技术新颖性", Proposition 4.1).  Keeping all B
decode slots busy (continuous refill) does not change how many tokens are
generated or how much attention work they need, but it packs that work into
fewer, more expensive decode steps.  A synchronous wave of B requests lasts as
long as its longest response, M_B = max of B response lengths, while under
ideal refill the B slots get through B requests in about E[L] steps; the
ratio C_KV = E[M_B] / E[L] is at least 1, grows with B, and equals 1 only for
a degenerate length law.  A slot observed at a random step holds a
length-biased response at a uniform position (inspection paradox), so the
mean context is P + (mu - 1)/2 + sigma^2 / (2 mu) (+1 for the token appended
at that step).

Model (readings; the pages give the law, not a simulator):
  * requests are i.i.d.: prompt P ~ U{p_lo..p_hi}, response length
    L = min(cap, max(1, ceil(X))) with X lognormal of the given mean and sd;
  * one decode step produces one token for every active request; request i,
    started at step s_i, is active at steps s_i .. s_i + L_i - 1, and at step t
    its context (including the token appended at t) is P_i + (t - s_i) + 1;
  * waves: requests [kB, (k+1)B) start together when the previous wave's
    longest response has finished;
  * refill: each request starts on the slot that frees first (list
    scheduling in arrival order), with no idle step;
  * page budget: pages of 16 positions; a waiting request is admitted to a
    free slot when its first step fits in the budget; when growth exceeds the
    budget the most recently admitted requests are preempted and requeued at
    the front, their generated tokens discarded (recompute on readmission).

This module holds scheduling only; none of the attention arithmetic.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np

from .lengths import RESPONSE_CAP, lognormal_moments_to_params

PAGE = 16


# ------------------------------------------------------------------ laws --

@dataclass
class LengthLaw:
    """Discrete response-length law on {1..cap} (pmf[l-1] = P(L = l)) and a
    uniform prompt law U{p_lo..p_hi}."""
    pmf: np.ndarray
    p_lo: int = 128
    p_hi: int = 512

    @classmethod
    def lognormal(cls, mean: float, sd: float, cap: int = RESPONSE_CAP, p_lo: int = 128,
                  p_hi: int = 512) -> "LengthLaw":
        """L = min(cap, max(1, ceil(X))), X lognormal with the given mean / sd."""
        from scipy.stats import lognorm
        m, s = lognormal_moments_to_params(mean, sd)
        edges = np.arange(0, cap + 1, dtype=np.float64)  # P(L <= l) = P(X <= l) for l < cap
        cdf = lognorm.cdf(edges, s, scale=math.exp(m))
        cdf[-1] = 1.0
        pmf = np.diff(cdf)
        return cls(pmf / pmf.sum(), p_lo, p_hi)

    @classmethod
    def uniform(cls, n: int, p_lo: int = 0, p_hi: int = 0) -> "LengthLaw":
        return cls(np.full(n, 1.0 / n), p_lo, p_hi)

    @classmethod
    def constant(cls, n: int, p_lo: int = 0, p_hi: int = 0) -> "LengthLaw":
        pmf = np.zeros(n)
        pmf[-1] = 1.0
        return cls(pmf, p_lo, p_hi)

    @property
    def support(self) -> np.ndarray:
        return np.arange(1, len(self.pmf) + 1, dtype=np.float64)

    def mean(self) -> float:
        return float((self.support * self.pmf).sum())

    def var(self) -> float:
        mu = self.mean()
        return float(((self.support - mu) ** 2 * self.pmf).sum())

    def prompt_mean(self) -> float:
        return 0.5 * (self.p_lo + self.p_hi)

    def expected_max(self, B: int) -> float:
        """E[M_B] = sum_l l (F(l)^B - F(l-1)^B) for B i.i.d. lengths."""
        F = np.cumsum(self.pmf)
        F = np.minimum(F, 1.0)
        Fm = np.concatenate([[0.0], F[:-1]])
        return float((self.support * (F ** B - Fm ** B)).sum())

    def draw(self, rng: np.random.Generator, n: int) -> tuple[np.ndarray, np.ndarray]:
        """n requests: (prompt lengths, response lengths), int64."""
        L = rng.choice(len(self.pmf), size=n, p=self.pmf) + 1
        P = rng.integers(self.p_lo, self.p_hi + 1, size=n)
        return P.astype(np.int64), L.astype(np.int64)


def kv_concentration(law: LengthLaw, B: int) -> float:
    """C_KV = E[M_B] / E[L] (Proposition 4.1)."""
    return law.expected_max(B) / law.mean()


def refill_mean_context(law: LengthLaw) -> float:
    """Mean context of an occupied slot under continuous refill, counting the
    token appended at that step: P + (mu - 1)/2 + sigma^2/(2 mu) + 1."""
    mu, var = law.mean(), law.var()
    return law.prompt_mean() + (mu - 1.0) / 2.0 + var / (2.0 * mu) + 1.0


# ------------------------------------------------------------- schedules --

@dataclass
class Schedule:
    """Start step of every request, with the request lengths it was built for."""
    policy: str
    B: int
    P: np.ndarray
    L: np.ndarray
    start: np.ndarray
    slot: np.ndarray
    steps: int = 0
    preempted_tokens: int = 0
    per_step: dict = field(default_factory=dict)

    def summary(self) -> dict:
        """Aggregates over all decode steps: tokens (one per active request per
        step), mean active batch, mean resident context (positions summed over
        active requests, per step), mean context per active request."""
        L, P = self.L.astype(np.float64), self.P.astype(np.float64)
        tokens = float(L.sum())
        ctx_steps = float((L * (P + 1.0) + L * (L - 1.0) / 2.0).sum())
        steps = float(self.steps)
        return dict(policy=self.policy, B=self.B, requests=int(len(L)), steps=int(self.steps),
                    tokens=int(tokens), mean_active=tokens / steps,
                    mean_resident_ctx=ctx_steps / steps, mean_ctx_per_active=ctx_steps / tokens,
                    preempted_tokens=int(self.preempted_tokens))

    def active_at(self, t: int) -> np.ndarray:
        """Indices of the requests active at step t."""
        return np.nonzero((self.start <= t) & (t < self.start + self.L))[0]

    def contexts_at(self, t: int) -> np.ndarray:
        """Contexts (including the token appended at step t) of the active requests."""
        i = self.active_at(t)
        return (self.P[i] + (t - self.start[i]) + 1).astype(np.int64)


def schedule_waves(P: np.ndarray, L: np.ndarray, B: int) -> Schedule:
    n = len(L)
    start = np.zeros(n, np.int64)
    slot = np.arange(n) % B
    t = 0
    for k in range(0, n, B):
        start[k:k + B] = t
        t += int(L[k:k + B].max())
    return Schedule("waves", B, P, L, start, slot, steps=t)


def schedule_refill(P: np.ndarray, L: np.ndarray, B: int) -> Schedule:
    """List scheduling in arrival order: each request takes the slot that
    frees first (ties: lowest slot)."""
    n = len(L)
    start = np.zeros(n, np.int64)
    slot = np.zeros(n, np.int64)
    heap = [(0, s) for s in range(B)]
    heapq.heapify(heap)
    end = 0
    for i in range(n):
        t, s = heapq.heappop(heap)
        start[i], slot[i] = t, s
        heapq.heappush(heap, (t + int(L[i]), s))
        end = max(end, t + int(L[i]))
    return Schedule("refill", B, P, L, start, slot, steps=end)


def pages_of(ctx) -> np.ndarray:
    return (np.asarray(ctx) + PAGE - 1) // PAGE


def simulate_paged(P: np.ndarray, L: np.ndarray, B: int, page_budget: int,
                   record: bool = False) -> Schedule:
    """Continuous refill under a KV page budget, one step at a time.  Returns
    the schedule of each request's final (completed) run; preempted work is
    counted in preempted_tokens.  record=True keeps per-step active counts,
    resident context and pages in use."""
    n = len(L)
    if pages_of(P.max() + 1) > page_budget:
        raise ValueError("a single prompt does not fit in the page budget")
    queue = list(range(n))[::-1]  # pop() takes the next request in arrival order
    slot_req = np.full(B, -1, np.int64)
    slot_pos = np.zeros(B, np.int64)
    slot_since = np.zeros(B, np.int64)  # admission step, for preemption order
    start = np.full(n, -1, np.int64)
    slot_of = np.zeros(n, np.int64)
    done = 0
    t = 0
    wasted = 0
    hist_active, hist_ctx, hist_pages = [], [], []
    while done < n:
        # admit waiting requests into free slots while their first step fits
        active = slot_req >= 0
        used = int(pages_of(P[slot_req[active]] + slot_pos[active] + 1).sum()) if active.any() else 0
        for s in np.nonzero(~active)[0]:
            if not queue:
                break
            i = queue[-1]
            need = int(pages_of(P[i] + 1))
            if used + need > page_budget:
                break
            queue.pop()
            slot_req[s], slot_pos[s], slot_since[s] = i, 0, t
            start[i] = t
            used += need
        active = slot_req >= 0
        # growth: preempt the most recently admitted requests until the step fits
        ctx = P[slot_req[active]] + slot_pos[active] + 1
        used = int(pages_of(ctx).sum())
        while used > page_budget:
            cand = np.nonzero(active)[0]
            s = cand[np.lexsort((-cand, -slot_since[cand]))[0]]
            i = slot_req[s]
            wasted += int(slot_pos[s])
            queue.append(i)
            start[i] = -1
            slot_req[s] = -1
            active = slot_req >= 0
            ctx = P[slot_req[active]] + slot_pos[active] + 1
            used = int(pages_of(ctx).sum())
        if record:
            hist_active.append(int(active.sum()))
            hist_ctx.append(int(ctx.sum()))
            hist_pages.append(used)
        # one decode step
        slot_pos[active] += 1
        fin = active & (slot_pos >= L[np.maximum(slot_req, 0)])
        for s in np.nonzero(fin)[0]:
            slot_of[slot_req[s]] = s
            slot_req[s] = -1
            done += 1
        t += 1
        if not active.any() and queue:
            raise RuntimeError("no request fits in the page budget")
    sch = Schedule("refill-paged", B, P, L, start, slot_of, steps=t, preempted_tokens=wasted)
    if record:
        sch.per_step = dict(active=np.array(hist_active), ctx=np.array(hist_ctx),
                            pages=np.array(hist_pages))
    return sch


# ---------------------------------------------------------------- replay --

def refill_snapshot(law: LengthLaw, B: int, seed: int, n_requests: int | None = None) -> np.ndarray:
    """Contexts of the B slots at one steady-state step of continuous refill
    (a replayable decode batch): enough requests that the sampled step lies
    well inside the run, the step drawn from the middle half."""
    rng = np.random.default_rng(seed)
    mu = law.mean()
    if n_requests is None:
        n_requests = int(B * (4 + 4 * len(law.pmf) / mu))
    P, L = law.draw(rng, n_requests)
    sch = schedule_refill(P, L, B)
    lo = int(len(law.pmf))  # past the first cap-length transient
    hi = int(sch.start.max())
    t = int(rng.integers(lo, max(lo + 1, hi)))
    ctx = sch.contexts_at(t)
    assert len(ctx) == B, (len(ctx), B)
    return ctx


def report(mean: float = 3000.0, sd: float = 2250.0, B_list=(1, 16, 64, 256, 512), n_per_slot: int = 60,
           seed: int = 0) -> list[dict]:
    """Waves against refill for one length law: closed-form C_KV and mean
    context, and the simulated steps, active batch and resident context."""
    law = LengthLaw.lognormal(mean, sd)
    rows = []
    for B in B_list:
        rng = np.random.default_rng(seed + B)
        P, L = law.draw(rng, B * n_per_slot)
        w, r = schedule_waves(P, L, B).summary(), schedule_refill(P, L, B).summary()
        rows.append(dict(B=B, C_KV=kv_concentration(law, B), waves_steps=w["steps"],
                         refill_steps=r["steps"], sim_ratio=w["steps"] / (w["tokens"] / B),
                         waves_active=w["mean_active"], refill_active=r["mean_active"],
                         waves_resident_ctx=w["mean_resident_ctx"],
                         refill_resident_ctx=r["mean_resident_ctx"],
                         mean_ctx=r["mean_ctx_per_active"], mean_ctx_law=refill_mean_context(law)))
    return rows


if __name__ == "__main__":
    import argparse
    import json
    ap = argparse.ArgumentParser(description="KV concentration: waves vs continuous refill")
    ap.add_argument("--mean", type=float, default=3000.0)
    ap.add_argument("--sd", type=float, default=2250.0)
    ap.add_argument("--B", type=int, nargs="*", default=[1, 16, 64, 256, 512])
    args = ap.parse_args()
    for row in report(args.mean, args.sd, tuple(args.B)):
        print(json.dumps({k: (round(v, 4) if isinstance(v, float) else v) for k, v in row.items()}))
