"""The one-launch decode step (kv4_append_decode_attention) against kv4_append
followed by kv4_decode_attention on copies of the same cache: out, lse, page
blocks and side rows bit-identical, for the default budget, other budgets
(w = 0 runs the append as its own launch) and inside a HIP graph."""
import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
from synth import make_workload
from tests.gpu_util import SCALE, GpuCase, bf, i32
from tests.wl import host_inputs

pytestmark = pytest.mark.gpu

EDGE = [1, 2, 15, 16, 17, 31, 143, 144, 145, 160, 161, 300, 1000]


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _clone(cache, sink, window):
    return kv4.Kv4Cache(cache.pages.clone(), cache.side_codes.clone(), cache.side_scales.clone(), sink, window)


@pytest.mark.parametrize("name,kw,sw", [
    ("edges_8_2", dict(ctx=EDGE, Hq=8, Hkv=2, seed=101), (16, 128)),
    ("short", dict(), (16, 128)),
    ("split_budget", dict(ctx=EDGE, Hq=4, Hkv=1, seed=102), (32, 64)),
    ("all_sink_fallback", dict(ctx=EDGE, Hq=4, Hkv=1, seed=103), (144, 0)),
    ("all_recent", dict(ctx=EDGE, Hq=4, Hkv=1, seed=104), (0, 144)),
    ("window_100", dict(ctx=EDGE, Hq=8, Hkv=2, seed=105), (16, 100)),
    ("window_7", dict(ctx=EDGE + [8, 23, 24, 25, 151, 152, 153], Hq=4, Hkv=1, seed=106), (0, 7)),
    ("window_1", dict(ctx=EDGE + [18, 33], Hq=4, Hkv=1, seed=107), (32, 1)),
])
def test_fused_step_equals_append_then_decode(name, kw, sw):
    _say(f"[fused] {name} s={sw[0]} w={sw[1]}")
    dev = torch.device("cuda")
    wl = make_workload(1 if name == "short" else 0, **kw)
    hi = host_inputs(wl)
    base = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev, *sw)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    if len(k):
        kv4.prefill_quantize(base, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev), slots, table,
                             int(max(1, lead.max())))
    ka, va = hi.at(lead)
    k_new, v_new, pos = bf(ka, dev), bf(va, dev), i32(lead, dev)
    q, ctx = bf(hi.q, dev), i32(wl.ctx, dev)
    a = _clone(base, *sw)
    b = _clone(base, *sw)
    kv4.append(a, k_new, v_new, pos, slots, table)
    o1, l1 = kv4.decode_attention(a, q, ctx, slots, table, wl.max_ctx, SCALE)
    o2, l2 = kv4.append_decode_attention(b, k_new, v_new, pos, q, ctx, slots, table, wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    assert torch.equal(a.pages, b.pages), "pages differ"
    assert torch.equal(a.side_codes, b.side_codes) and torch.equal(a.side_scales, b.side_scales)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fused_step_in_a_graph():
    _say("[fused] graph capture, 5 replays")
    dev = torch.device("cuda")
    wl = make_workload(1)
    hi = host_inputs(wl)
    case = GpuCase(wl, hi)
    ka, va = hi.at(wl.ctx - 1)
    k_new, v_new, pos = bf(ka, dev), bf(va, dev), i32(wl.ctx - 1, dev)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(kv4.decode_workspace_bytes(case.cache, wl.B, wl.Hq, wl.max_ctx), dtype=torch.uint8, device=dev)

    def step():
        kv4.append_decode_attention(case.cache, k_new, v_new, pos, case.q, case.ctx, case.slots, case.table,
                                    wl.max_ctx, SCALE, out, lse, ws)

    step()
    torch.cuda.synchronize()
    ref_out, ref_lse, ref_pages = out.clone(), lse.clone(), case.cache.pages.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(5):
        out.fill_(float("nan"))
        ws.fill_(0x5A)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse), rep
        assert torch.equal(case.cache.pages, ref_pages), rep
