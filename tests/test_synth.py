"""Pins of the synthetic workload generator: the length-biased context law
against the pages' closed form, and page-table validity."""
import numpy as np
import pytest

from synth import CONFIGS, law_mean_context, make_workload, sample_contexts


@pytest.mark.parametrize("mean,sd", [(4000.0, 3000.0), (1450.0, 1087.5), (3000.0, 2250.0)])
def test_length_biased_mean_context_closed_form(mean, sd):
    # mean context seen by a decode step: P + (mu-1)/2 + sigma^2/(2 mu); our
    # contexts also count this step's token (+1); the 16,383-position cap
    # costs about 1.2% at mu = 4k, inside the 2% allowance.
    rng = np.random.default_rng(2024)
    ctx = sample_contexts(rng, 1_000_000, mean, sd)
    want = law_mean_context(mean, sd)
    assert abs((ctx - 1).mean() - want) <= 0.02 * want
    assert ctx.min() >= 129 and ctx.max() <= 512 + 16383 + 1


def test_uncapped_law_matches_closed_form_tightly():
    rng = np.random.default_rng(3)
    ctx = sample_contexts(rng, 2_000_000, 1000.0, 500.0, cap=10 ** 9)
    want = law_mean_context(1000.0, 500.0)
    assert abs((ctx - 1).mean() - want) <= 0.003 * want


@pytest.mark.parametrize("index", sorted(CONFIGS))
def test_workload_page_tables(index):
    wl = make_workload(index)
    assert wl.B == CONFIGS[index]["B"]
    need = (wl.ctx + 15) // 16
    used = np.concatenate([wl.page_table[b, :need[b]] for b in range(wl.B)])
    assert len(np.unique(used)) == len(used)           # no page shared
    assert used.min() >= 0 and used.max() < wl.num_pages
    if index == 0:
        assert list(wl.ctx) == [100, 144, 400, 700] and wl.num_pages == 128 and wl.pt_stride == 64
    if index == 3:
        assert wl.ctx.min() >= 12000 and wl.ctx.max() <= 16896
        assert wl.num_pages == need.sum()              # zero-slack pool
