"""GPU parity of the protection-budget variants (s sink positions, w recent
positions): unprotected KV4 (s = w = 0), all-sink (s = 144), all-recent
(w = 144) and an intermediate split (s = 32, w = 64), against the oracle run
with the same budget.  Same bar as the default budget: cache bytes, query
codes, int32 QK / PV accumulators and P-operand codes bit-exact, out within
2e-3 and lse within 1e-4."""
import pytest
import torch

from synth import make_workload
from tests.gpu_util import GpuCase
from tests.test_gpu_parity import assert_cache_equal, assert_decode_matches
from tests.wl import host_inputs, oracle_cache

pytestmark = pytest.mark.gpu

BUDGETS = [(0, 0), (144, 0), (0, 144), (32, 64)]
# every boundary of the four budgets: s, s+1, L-w around page edges, 144
EDGE = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 95, 96, 97, 143, 144, 145, 159, 160, 161, 177,
        300, 1000]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("s,w", BUDGETS, ids=[f"s{s}w{w}" for s, w in BUDGETS])
def test_budget_parity_edges(s, w):
    _say(f"[budget] s={s} w={w} edge contexts, Hq=8 Hkv=2")
    wl = make_workload(0, ctx=EDGE, Hq=8, Hkv=2, seed=31)
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi, sink=s, window=w)
    case = GpuCase(wl, hi, sink=s, window=w)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    err, lerr = assert_decode_matches(case, ref)
    _say(f"[budget] s={s} w={w}: out {err:.2e} lse {lerr:.2e}")


@pytest.mark.parametrize("s,w", BUDGETS, ids=[f"s{s}w{w}" for s, w in BUDGETS])
def test_budget_appends_equal_prefill(s, w):
    _say(f"[budget] s={s} w={w} appends == prefill")
    wl = make_workload(0, ctx=EDGE[::3], Hq=4, Hkv=1, seed=32)
    hi = host_inputs(wl)
    a = GpuCase(wl, hi, use_prefill=False, sink=s, window=w)
    b = GpuCase(wl, hi, use_prefill=True, sink=s, window=w)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.pages, b.cache.pages)
    assert torch.equal(a.cache.side_codes, b.cache.side_codes)
    assert torch.equal(a.cache.side_scales, b.cache.side_scales)


def test_unprotected_short_workload():
    """s = w = 0 on the 64-sequence short workload: every position in the
    integer path, many chunks per segment."""
    _say("[budget] s=0 w=0 short workload B=64")
    wl = make_workload(1)
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi, sink=0, window=0)
    case = GpuCase(wl, hi, sink=0, window=0)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    err, lerr = assert_decode_matches(case, ref)
    _say(f"[budget] unprotected short: out {err:.2e} lse {lerr:.2e}")
