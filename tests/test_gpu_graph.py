"""The library's launches captured in a HIP graph (append + decode of one
layer) replay to the same bytes as the eager calls, replay after replay,
with unrelated eager work and synchronizations between the replays."""
import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
from synth import make_workload
from tests.gpu_util import SCALE, GpuCase, bf, i32
from tests.wl import host_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def test_graph_replays_match_eager():
    print("[graph] short workload, append + decode captured", flush=True)
    wl = make_workload(1)
    hi = host_inputs(wl)
    case = GpuCase(wl, hi)  # cache holds positions [0, ctx-1) and this step's token
    dev = case.dev
    ka, va = hi.at(wl.ctx - 1)
    k_app, v_app, pos = bf(ka, dev), bf(va, dev), i32(wl.ctx - 1, dev)
    out = torch.empty((wl.B, wl.Hq, 128), dtype=torch.float32, device=dev)
    lse = torch.empty((wl.B, wl.Hq), dtype=torch.float32, device=dev)
    ws = torch.empty(kv4.decode_workspace_bytes(case.cache, wl.B, wl.Hq, wl.max_ctx), dtype=torch.uint8,
                     device=dev)

    def layer_step():
        # re-appending the same token rewrites the same bytes
        kv4.append(case.cache, k_app, v_app, pos, case.slots, case.table)
        kv4.decode_attention(case.cache, case.q, case.ctx, case.slots, case.table, wl.max_ctx, SCALE,
                             out, lse, ws)

    layer_step()
    torch.cuda.synchronize()
    ref_out, ref_lse = out.clone(), lse.clone()
    ref_pages = case.cache.pages.clone()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer_step()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer_step()
    torch.cuda.synchronize()

    scratch = torch.randn(1 << 20, device=dev)
    for rep in range(5):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        ws.fill_(0xA5)  # stale workspace must not matter
        scratch.mul_(1.0001).add_(1.0)  # unrelated eager work
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out), f"replay {rep}: out differs"
        assert torch.equal(lse, ref_lse), f"replay {rep}: lse differs"
        assert torch.equal(case.cache.pages, ref_pages), f"replay {rep}: pages differ"
        # an eager call between replays, into other buffers
        o2, l2 = case.decode()
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_out) and torch.equal(l2, ref_lse)
    print("[graph] 5 replays bit-identical to eager", flush=True)
