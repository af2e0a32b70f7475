"""Group sizes other than 4 on the GPU against the oracle: G = Hq / Hkv query
heads per kv-head with G in {1, 2, 3, 5, 8, 16} (one partial virtual group of
query heads when G % 4 != 0; two groups when G = 5 or 8, four when G = 16).  The kernels' rows
are groups of at most 4 query heads of one kv-head; the oracle maps query
head h to kv-head h // G directly, so a wrong head-to-group mapping, a row
past a group's last head that is stored, or a group that appends a kv-head
twice fails here.  Covered: the decode (debug intermediates), the one-launch
step with this step's append, re-prefill attention (debug intermediates), the
MXFP4 format and KV8 everywhere, each with a random budget.  Bar: page blocks,
side rows, query codes and sums, int32 QK, P codes and int32 PV bit-exact; out
within 2e-3 max-abs, lse within 1e-4."""
import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
import oracle
from synth import make_workload
from tests.gpu_util import SCALE, GpuCase, bf, i32
from tests.test_gpu_parity import assert_cache_equal
from tests.test_gpu_random import BUDGETS, EDGES, ODD_BUDGETS, _compare
from tests.wl import host_inputs, oracle_cache

pytestmark = pytest.mark.gpu

OUT_TOL, LSE_TOL = 2e-3, 1e-4
GROUPS = [1, 2, 3, 5, 8, 16]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _workload(G, seed):
    """A tiny-config workload with G query heads per kv-head, random batch,
    kv-head count, contexts (half on region edges), slots, pool and budget."""
    rng = np.random.default_rng(9000 + 17 * G + seed)
    B = int(rng.integers(1, 14))
    Hkv = int(rng.choice([1, 2, 3]))
    ctx = np.where(rng.random(B) < 0.5, rng.choice(EDGES, B), rng.integers(1, 900, B))
    wl = make_workload(0, seed=9500 + 17 * G + seed, ctx=ctx, Hq=G * Hkv, Hkv=Hkv,
                       pool_slack=int(rng.integers(1, 16)))
    extra = int(rng.integers(0, 4))
    wl.slots = rng.permutation(B + extra)[:B].astype(np.int32)
    wl.max_slots = B + extra
    pool = BUDGETS + ODD_BUDGETS
    sink, window = pool[int(rng.integers(0, len(pool)))]
    return wl, sink, window


def _tag(kind, G, seed, wl, sink, window):
    return f"{kind} G={G} seed {seed} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} s={sink} w={window} " \
           f"ctx max {int(wl.ctx.max())}"


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("G", GROUPS)
def test_gqa_decode(G, seed):
    wl, sink, window = _workload(G, seed)
    tag = _tag("decode", G, seed, wl, sink, window)
    _say(f"[gqa] {tag}")
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi, sink=sink, window=window)
    case = GpuCase(wl, hi, sink=sink, window=window)
    out, lse, dbg = case.decode(debug=True)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    r_out, r_lse, r_dbg = oracle.decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq,
                                        SCALE, debug=True)
    _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg)
    # the release launch gives the debug launch's outputs
    out2, lse2 = kv4.decode_attention(case.cache, bf(hi.q, case.dev), i32(wl.ctx, case.dev), case.slots,
                                      case.table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2), tag


@pytest.mark.parametrize("seed", range(2))
@pytest.mark.parametrize("G", GROUPS)
def test_gqa_fused_step(G, seed):
    """The one-launch step: the kv-head's first head group appends this step's
    token, every group patches its side row; pages, side rows, out and lse
    against the oracle's append followed by its decode."""
    wl, sink, window = _workload(G, 10 + seed)
    tag = _tag("fused", G, seed, wl, sink, window)
    _say(f"[gqa] {tag}")
    dev = torch.device("cuda")
    hi = host_inputs(wl)
    ref = oracle_cache(wl, hi, sink=sink, window=window)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, sink, window)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    if len(k):
        kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev), slots, table,
                             int(max(1, lead.max())))
    ka, va = hi.at(lead)
    out, lse = kv4.append_decode_attention(cache, bf(ka, dev), bf(va, dev), i32(lead, dev), bf(hi.q, dev),
                                           i32(wl.ctx, dev), slots, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert np.array_equal(cache.pages.cpu().numpy(), ref.pages), tag
    assert np.array_equal(cache.side_codes.cpu().numpy(), ref.side_codes), tag
    assert np.array_equal(cache.side_scales.cpu().numpy().view(np.uint16), ref.side_scales.view(np.uint16)), tag
    r_out, r_lse, _ = oracle.decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[gqa] {tag}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


@pytest.mark.parametrize("G", GROUPS)
def test_gqa_prefill_attention(G):
    """Chunks of random length at the end of each prefix (causal inside the
    chunk), debug intermediates bit-exact."""
    rng = np.random.default_rng(9900 + G)
    wl, sink, window = _workload(G, 20)
    n = np.minimum(wl.ctx, rng.integers(1, 70, wl.B)).astype(np.int32)
    tag = _tag("re-prefill", G, 20, wl, sink, window) + f" tokens {int(n.sum())}"
    _say(f"[gqa] {tag}")
    dev = torch.device("cuda")
    hi = host_inputs(wl)
    k, v, cu_all = hi.prefix(wl.ctx)
    ref = oracle.Cache(wl.num_pages, wl.Hkv, wl.max_slots, sink, window)
    oracle.prefill(ref, k, v, cu_all, np.zeros(wl.B, np.int32), wl.slots, wl.page_table)
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, sink, window)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu_all, dev), i32(np.zeros(wl.B), dev), slots, table,
                         int(wl.ctx.max()))
    start = (wl.ctx - n).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    T = int(cu[-1])
    qr = np.random.default_rng(9950 + G).standard_normal((T, wl.Hq, 128)).astype(np.float32)
    q = torch.from_numpy(qr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out, lse, dbg = kv4.prefill_attention_debug(cache, bf(q, dev), i32(cu, dev), i32(start, dev), slots, table,
                                                int(wl.ctx.max()), SCALE)
    out2, lse2 = kv4.prefill_attention(cache, bf(q, dev), i32(cu, dev), i32(start, dev), slots, table,
                                       int(wl.ctx.max()), SCALE)
    torch.cuda.synchronize()
    r_out, r_lse, r_dbg = oracle.prefill_attention(ref, q, cu, start, wl.slots, wl.page_table, wl.Hq, SCALE,
                                                   debug=True)
    _compare(tag, out, lse, dbg, r_out, r_lse, r_dbg)
    assert torch.equal(out, out2) and torch.equal(lse, lse2), tag


@pytest.mark.parametrize("G", GROUPS)
def test_gqa_mx(G):
    from tests.test_gpu_mx import _Case, _oracle_mx
    wl, sink, window = _workload(G, 30)
    tag = _tag("mxfp4", G, 30, wl, sink, window)
    _say(f"[gqa] {tag}")
    dev = torch.device("cuda")
    hi = host_inputs(wl)
    ref = _oracle_mx(wl, hi, sink, window)
    case = _Case(wl, hi, sink, window, dev)
    out, lse = kv4.mx_decode_attention(case.cache, bf(hi.q, dev), i32(wl.ctx, dev), case.slots, case.table,
                                       wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert_cache_equal(case, ref)
    r_out, r_lse = oracle.mx_decode(ref, hi.q, wl.ctx.astype(np.int32), wl.slots, wl.page_table, wl.Hq, SCALE)
    err = float(np.abs(out.cpu().numpy() - r_out).max())
    lerr = float(np.abs(lse.cpu().numpy() - r_lse).max())
    _say(f"[gqa] {tag}: out {err:.2e} lse {lerr:.2e}")
    assert err <= OUT_TOL and lerr <= LSE_TOL, (tag, err, lerr)


@pytest.mark.parametrize("G", GROUPS)
def test_gqa_kv8(G):
    from tests.test_gpu_kv8 import _check
    wl, _, _ = _workload(G, 40)
    tag = f"kv8 G={G} B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} ctx max {int(wl.ctx.max())}"
    _say(f"[gqa] {tag}")
    err, lerr = _check(wl, host_inputs(wl), torch.device("cuda"))
    _say(f"[gqa] {tag}: out {err:.2e} lse {lerr:.2e}")


def test_gqa_comparator_refuses_other_groups():
    """The BF16 comparator keeps exactly 4 query heads per kv-head."""
    dev = torch.device("cuda")
    pages = torch.zeros((4, 2, 2, 16, 128), dtype=torch.bfloat16, device=dev)
    q = torch.zeros((1, 6, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(kv4.Kv4Error):
        kv4.bf16_paged_decode(pages, q, torch.ones(1, dtype=torch.int32, device=dev),
                              torch.zeros((1, 1), dtype=torch.int32, device=dev), 16, SCALE)
