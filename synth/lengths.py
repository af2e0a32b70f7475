"""Context-length laws for synthetic decode batches.

KV concentration (onedev.kr summary, "어떻게 동작하나"; paper.rainbus.top
summary, "研究动机", Prop. 4.1): under continuous refill a decode slot is more
likely to be occupied by a long response (inspection paradox), so the response
length seen at a decode step is length-biased, and the position inside it is
uniform.  The pages give the resulting mean context as P + (mu-1)/2 +
sigma^2/(2 mu), with P the prompt length and mu, sigma the mean and standard
deviation of the response length.

Readings (the pages are silent on the exact sampler):
  * mu and sigma are the mean and standard deviation of the response length L
    itself; the lognormal parameters follow from them.
  * The length-biased law of a lognormal(m, s) is lognormal(m + s^2, s).
  * The position r inside the sampled response is uniform on {0..ceil(L*)-1},
    capped at 16383 (the 16,384-token response cap); the context handed to the
    kernels counts the token appended this step, ctx = P + r + 1.
"""
from __future__ import annotations

import math

import numpy as np

RESPONSE_CAP = 16384


def lognormal_moments_to_params(mean: float, sd: float) -> tuple[float, float]:
    """Return (m, s) of ln L for a lognormal L with the given mean and sd."""
    s2 = math.log1p((sd / mean) ** 2)
    return math.log(mean) - 0.5 * s2, math.sqrt(s2)


def sample_contexts(rng: np.random.Generator, n: int, mean: float, sd: float,
                    p_lo: int = 128, p_hi: int = 512,
                    cap: int = RESPONSE_CAP - 1) -> np.ndarray:
    """Draw n context lengths (including this step's token) from the
    length-biased lognormal response law plus a uniform prompt length."""
    m, s = lognormal_moments_to_params(mean, sd)
    l_star = rng.lognormal(m + s * s, s, size=n)
    r = np.floor(rng.random(n) * np.ceil(l_star)).astype(np.int64)
    r = np.minimum(r, cap)
    prompt = rng.integers(p_lo, p_hi + 1, size=n)
    return (prompt + r + 1).astype(np.int64)


def law_mean_context(mean: float, sd: float, p_lo: int = 128, p_hi: int = 512) -> float:
    """Closed-form mean context before this step's token, P + (mu-1)/2 + sigma^2/(2 mu)."""
    p_bar = 0.5 * (p_lo + p_hi)
    return p_bar + (mean - 1.0) / 2.0 + sd * sd / (2.0 * mean)
