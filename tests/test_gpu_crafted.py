"""GPU parity on hand-made pages (raw bytes written directly, no quantizer)
for degenerate cases of the main-region P-operand rule, decode and
re-prefill attention.  Bar as elsewhere: query codes and sums, int32 QK, P
codes and int32 PV bit-exact; out within 2e-3 max-abs, lse within 1e-4."""
import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from tests import crafted
from tests.gpu_util import SCALE, bf, i32

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg):
    for key in ("qcodes", "qsum", "qk", "pcode", "pv"):
        got = dbg[key].cpu().numpy()
        bad = np.argwhere(got != r_dbg[key])
        assert len(bad) == 0, f"{tag} {key}: {len(bad)} mismatches, first {bad[:4].tolist()}"
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    print(f"[crafted] {tag}: out {err:.2e} lse {lerr:.2e}", flush=True)
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


@pytest.mark.parametrize("name", sorted(crafted.CASES))
def test_crafted_page(name):
    """u_max_subnormal: u_max FP32-subnormal and 127 / u_max infinite, so the
    nonzero u saturate at 127 and the zero weight gives code 0 (FP32
    subnormals kept through the weights, the products and the division);
    weights_cut_off: weights below the exp2s cutoff are exactly 0;
    u_max_zero: constant V vectors, every code 0."""
    dev = torch.device("cuda")
    ref = oracle.Cache(2, 1, 1, sink=0, window=0)
    ref.pages[0, 0] = crafted.page(name)
    cache = kv4.Kv4Cache.zeros(2, 1, 1, dev, 0, 0)
    cache.pages.copy_(torch.from_numpy(ref.pages))
    q = crafted.unit_query(1, 4)
    table, ctx, slot = np.array([[0, 1]], np.int32), np.array([16], np.int32), np.array([0], np.int32)
    print(f"[crafted] {name}: decode, one page, s = w = 0", flush=True)
    out, lse, dbg = kv4.decode_attention_debug(cache, bf(q, dev), i32(ctx, dev), i32(slot, dev),
                                               i32(table, dev), 32, SCALE)
    out2, lse2 = kv4.decode_attention(cache, bf(q, dev), i32(ctx, dev), i32(slot, dev), i32(table, dev), 32,
                                      SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    r_out, r_lse, r_dbg = oracle.decode(ref, q, ctx, slot, table, 4, SCALE, debug=True)
    _compare(f"{name} decode", out, lse, dbg, r_out, r_lse, r_dbg)
    print(f"[crafted] {name}: re-prefill attention, one-token chunk at position 15", flush=True)
    cu, start = np.array([0, 1], np.int32), np.array([15], np.int32)
    out, lse, dbg = kv4.prefill_attention_debug(cache, bf(q, dev), i32(cu, dev), i32(start, dev),
                                                i32(slot, dev), i32(table, dev), 32, SCALE)
    torch.cuda.synchronize()
    r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, slot, table, 4, SCALE, debug=True)
    _compare(f"{name} re-prefill", out, lse, dbg, r_out, r_lse, r_dbg)
