"""Pins of the KV-concentration simulator (CPU): Proposition 4.1 of the KV4-RL
pages (C_KV = E[M_B]/E[L] >= 1, nondecreasing in B), the inspection-paradox
mean context P + (mu-1)/2 + sigma^2/(2 mu), closed forms for E[M_B], and the
schedules' invariants (work conservation, page budget)."""
import math
from fractions import Fraction

import numpy as np
import pytest

from synth import make_workload, sample_contexts
from synth.concentration import (LengthLaw, kv_concentration, pages_of, refill_mean_context,
                                 refill_snapshot, schedule_refill, schedule_waves, simulate_paged)


def test_expected_max_uniform_closed_form():
    """U{1..n}: E[M_B] = sum_{k=0}^{n-1} (1 - (k/n)^B), in exact rationals."""
    for n, B in ((1, 5), (7, 1), (10, 3), (64, 16), (300, 256)):
        law = LengthLaw.uniform(n)
        want = sum(1 - Fraction(k, n) ** B for k in range(n))
        assert abs(law.expected_max(B) - float(want)) <= 1e-9 * float(want)


def test_expected_max_geometric_closed_form():
    """Geometric lengths P(L = l) = p q^(l-1): E[M_B] = sum_{j=1}^B C(B,j) (-1)^(j+1) / (1 - q^j)."""
    p = 0.05
    q = 1 - p
    n = 2000  # truncation mass q^2000 ~ 1e-45
    l = np.arange(1, n + 1)
    law = LengthLaw(p * q ** (l - 1.0))
    for B in (1, 2, 8, 32):
        want = sum(math.comb(B, j) * (-1) ** (j + 1) / (1 - q ** j) for j in range(1, B + 1))
        assert abs(law.expected_max(B) - want) < 1e-6 * want


def test_concentration_properties():
    law = LengthLaw.lognormal(3000, 2250)
    assert abs(kv_concentration(law, 1) - 1.0) < 1e-12
    c = [kv_concentration(law, B) for B in (1, 2, 4, 16, 64, 256, 512)]
    assert all(b >= a for a, b in zip(c, c[1:]))
    assert c[-1] > 1.0
    const = LengthLaw.constant(700)
    for B in (1, 8, 256):
        assert abs(kv_concentration(const, B) - 1.0) < 1e-12


@pytest.fixture(scope="module")
def small_law():
    return LengthLaw.lognormal(300, 250, cap=2048)


def test_waves_last_as_long_as_the_expected_max(small_law):
    rng = np.random.default_rng(1)
    B = 64
    P, L = small_law.draw(rng, 64 * 400)
    w = schedule_waves(P, L, B)
    assert abs(w.steps / 400 - small_law.expected_max(B)) < 0.015 * small_law.expected_max(B)


def test_refill_is_work_conserving(small_law):
    rng = np.random.default_rng(2)
    B = 32
    P, L = small_law.draw(rng, 3000)
    r = schedule_refill(P, L, B)
    assert (r.start[:B] == 0).all()
    # on every slot the requests follow each other without a gap
    for s in range(B):
        i = np.nonzero(r.slot == s)[0]
        assert (r.start[i[1:]] == r.start[i[:-1]] + L[i[:-1]]).all()
    # a request never waits while a slot is idle: it starts at the earliest slot release
    ideal = L.sum() / B
    assert ideal <= r.steps <= ideal + len(small_law.pmf)
    # never more than B active
    for t in np.linspace(0, r.steps - 1, 50).astype(int):
        assert len(r.active_at(int(t))) <= B


def test_concentration_ratio_from_the_schedules(small_law):
    """Waves need C_KV times the steps of ideal refill for the same tokens."""
    rng = np.random.default_rng(3)
    for B in (8, 64):
        P, L = small_law.draw(rng, B * 400)
        w = schedule_waves(P, L, B)
        ratio = w.steps / (L.sum() / B)
        assert abs(ratio - kv_concentration(small_law, B)) < 0.03 * kv_concentration(small_law, B)
        # the same tokens, so resident context per step scales by the same factor
        r = schedule_refill(P, L, B)
        sw, sr = w.summary(), r.summary()
        assert sw["tokens"] == sr["tokens"]
        assert sr["mean_resident_ctx"] / sw["mean_resident_ctx"] == pytest.approx(w.steps / r.steps)


def test_refill_mean_context_is_length_biased(small_law):
    rng = np.random.default_rng(4)
    B = 64
    P, L = small_law.draw(rng, 40000)
    r = schedule_refill(P, L, B)
    want = refill_mean_context(small_law)
    assert abs(r.summary()["mean_ctx_per_active"] - want) < 0.01 * want
    # snapshots of the steady state: the mean context of occupied slots
    ts = np.linspace(len(small_law.pmf), r.start.max(), 200).astype(int)
    snap = np.concatenate([r.contexts_at(int(t)) for t in ts])
    assert abs(snap.mean() - want) < 0.015 * want
    # the plain (not length-biased) mean would be far lower
    naive = small_law.prompt_mean() + (small_law.mean() - 1) / 2 + 1
    assert want - naive > 0.2 * small_law.var() / small_law.mean()


def test_snapshot_matches_the_length_biased_sampler():
    """A replayed refill batch and the closed-form length-biased sampler used
    for the benchmark workloads describe the same law."""
    law = LengthLaw.lognormal(3000, 2250)
    snaps = np.concatenate([refill_snapshot(law, 256, seed) for seed in range(12)])
    direct = sample_contexts(np.random.default_rng(9), 200000, 3000, 2250)
    assert abs(snaps.mean() - direct.mean()) < 0.03 * direct.mean()
    assert abs(snaps.mean() - refill_mean_context(law)) < 0.03 * refill_mean_context(law)


def test_page_budget():
    law = LengthLaw.lognormal(200, 150, cap=1024, p_lo=16, p_hi=64)
    rng = np.random.default_rng(5)
    B = 32
    P, L = law.draw(rng, 400)
    free = simulate_paged(P, L, B, page_budget=10 ** 9)
    ref = schedule_refill(P, L, B)
    assert free.steps == ref.steps and (free.start == ref.start).all()
    assert free.preempted_tokens == 0
    unconstrained = simulate_paged(P, L, B, page_budget=10 ** 9, record=True).per_step["pages"].max()
    tp = {}
    for frac in (1.0, 0.5, 0.25):
        budget = max(int(unconstrained * frac), int(pages_of(P.max() + 1)) + 1)
        s = simulate_paged(P, L, B, page_budget=budget, record=True)
        assert s.per_step["pages"].max() <= budget
        assert s.per_step["active"].max() <= B
        assert (s.start >= 0).all()  # every request completed
        tp[frac] = L.sum() / s.steps
    assert tp[0.25] < tp[0.5] <= tp[1.0] * 1.0001


def test_snapshot_replays_as_a_workload():
    law = LengthLaw.lognormal(3000, 2250)
    ctx = refill_snapshot(law, 256, 7)
    assert len(ctx) == 256 and ctx.min() >= 129 and ctx.max() <= 512 + 16384
    wl = make_workload(4, ctx=ctx)
    assert np.array_equal(wl.ctx, ctx) and wl.page_table.shape[0] == 256
