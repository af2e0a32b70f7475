"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Bar: INT4/INT8 codes, packed pages, side rows, query codes, int32 QK and PV
accumulators and P-operand codes bit-exact; attention output within 2e-3
max-abs and LSE within 1e-4 absolute."""
import numpy as np
import pytest
import torch

import oracle
from synth import make_workload
from tests.gpu_util import SCALE, GpuCase
from tests.wl import host_inputs, oracle_cache

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def assert_cache_equal(case, ref):
    pages = case.cache.pages.cpu().numpy()
    side = case.cache.side_codes.cpu().numpy()
    scales = case.cache.side_scales.cpu().numpy().view(np.uint16)
    bad = np.argwhere(pages != ref.pages)
    assert len(bad) == 0, f"{len(bad)} page bytes differ, first {bad[:4].tolist()}"
    assert np.array_equal(side, ref.side_codes), "side codes differ"
    assert np.array_equal(scales, ref.side_scales), "side scales differ"


def assert_decode_matches(case, ref_cache, check_debug=True):
    wl, hi = case.wl, case.hi
    out_d, lse_d, dbg = case.decode(debug=True)
    out, lse = case.decode()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_dbg = oracle.decode(ref_cache, hi.q, wl.ctx.astype(np.int32), wl.slots,
                                              wl.page_table, wl.Hq, SCALE, debug=True)
    # the debug instantiation only adds stores
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    if check_debug:
        for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
            got = dbg[key].cpu().numpy()
            want = ref_dbg[key]
            bad = np.argwhere(got != want)
            assert len(bad) == 0, f"{key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    err = np.abs(out.cpu().numpy() - ref_out).max()
    lerr = np.abs(lse.cpu().numpy() - ref_lse).max()
    assert err <= OUT_TOL, err
    assert lerr <= LSE_TOL, lerr
    return err, lerr


EDGE = [1, 2, 15, 16, 17, 143, 144, 145, 146, 159, 160, 161, 162, 175, 176, 177, 300, 1000]


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict()),
    ("edges_4_1", dict(ctx=EDGE, Hq=4, Hkv=1)),
    ("edges_8_2", dict(ctx=EDGE[::-1], Hq=8, Hkv=2, seed=3)),
])
def test_small_parity(name, kw):
    _say(f"[parity] {name}")
    wl = make_workload(0, **kw)
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi)
    case = GpuCase(wl, hi)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    err, lerr = assert_decode_matches(case, ref)
    _say(f"[parity] {name}: out {err:.2e} lse {lerr:.2e}")


def test_appends_equal_prefill():
    _say("[parity] appends == prefill")
    wl = make_workload(0, ctx=EDGE, Hq=4, Hkv=1, seed=5)
    hi = host_inputs(wl)
    a = GpuCase(wl, hi, use_prefill=False)
    b = GpuCase(wl, hi, use_prefill=True)
    torch.cuda.synchronize()
    assert torch.equal(a.cache.pages, b.cache.pages)
    assert torch.equal(a.cache.side_codes, b.cache.side_codes)
    assert torch.equal(a.cache.side_scales, b.cache.side_scales)


def test_short_workload_full_parity():
    _say("[parity] short B=64 32/8")
    wl = make_workload(1)
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi)
    case = GpuCase(wl, hi)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    err, lerr = assert_decode_matches(case, ref)
    _say(f"[parity] short: out {err:.2e} lse {lerr:.2e}")
