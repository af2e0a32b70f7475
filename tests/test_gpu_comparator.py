"""GPU checks of the BF16 paged-decode comparator (not part of the method) and
of the benchmark's timed decode entry point."""
import math

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


def bf16_pool(wl, hi, dev):
    """BF16 pages: per (page, kv-head) K token-major [16][128], V channel-major [128][16]."""
    pool = np.zeros((wl.num_pages, wl.Hkv, 2, 16, 128), np.uint16)
    for b in range(wl.B):
        for p in range(int(wl.ctx[b])):
            pg, t = wl.page_table[b, p // 16], p % 16
            pool[pg, :, 0, t, :] = hi.k[hi.offsets[b] + p]
            vt = pool[pg, :, 1].reshape(wl.Hkv, 128, 16)
            vt[:, :, t] = hi.v[hi.offsets[b] + p]
            pool[pg, :, 1] = vt.reshape(wl.Hkv, 16, 128)
    return bf(pool, dev)


def reference(wl, hi):
    f = lambda x: (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    out = np.zeros((wl.B, wl.Hq, 128))
    lse = np.zeros((wl.B, wl.Hq))
    for b in range(wl.B):
        K = f(hi.k[hi.offsets[b]:hi.offsets[b + 1]])  # [L][Hkv][128]
        V = f(hi.v[hi.offsets[b]:hi.offsets[b + 1]])
        for h in range(wl.Hq):
            g = h // wl.group
            z = K[:, g] @ f(hi.q[b, h]) * SCALE
            w = np.exp(z - z.max())
            out[b, h] = (w[:, None] * V[:, g]).sum(0) / w.sum()
            lse[b, h] = z.max() + math.log(w.sum())
    return out, lse


@pytest.mark.parametrize("index,kw", [(0, dict(ctx=[1, 15, 16, 17, 33, 145, 700], Hq=4, Hkv=1)),
                                      (1, dict())])
def test_bf16_comparator_matches_fp64_attention(index, kw):
    print(f"[comparator] workload {index}", flush=True)
    dev = torch.device("cuda")
    wl = make_workload(index, **kw)
    hi = host_inputs(wl)
    pool = bf16_pool(wl, hi, dev)
    out, lse = kv4.bf16_paged_decode(pool, bf(hi.q, dev), i32(wl.ctx, dev), i32(wl.page_table, dev),
                                     wl.max_ctx, SCALE)
    torch.cuda.synchronize()
    ref_out, ref_lse = reference(wl, hi)
    # P is rounded to BF16 for the MFMA: ~2^-9 relative per weight
    assert np.abs(out.cpu().numpy() - ref_out).max() < 2e-2
    assert np.abs(lse.cpu().numpy() - ref_lse).max() < 1e-3


def test_timed_entry_point_matches_decode():
    import ctypes
    dev = torch.device("cuda")
    wl = make_workload(0)
    hi = host_inputs(wl)
    case = GpuCase(wl, hi)
    out0, lse0 = case.decode()
    hip = ctypes.CDLL("libamdhip64.so")
    e0, e1 = ctypes.c_void_p(), ctypes.c_void_p()
    assert hip.hipEventCreate(ctypes.byref(e0)) == 0 and hip.hipEventCreate(ctypes.byref(e1)) == 0
    out = torch.empty_like(out0)
    lse = torch.empty_like(lse0)
    ws = torch.empty(kv4.decode_workspace_bytes(case.cache, wl.B, wl.Hq, wl.max_ctx),
                     dtype=torch.uint8, device=dev)
    kv4.decode_attention_timed(case.cache, case.q, case.ctx, case.slots, case.table, wl.max_ctx,
                               SCALE, out, lse, ws, e0, e1)
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), e0, e1) == 0 and ms.value >= 0
    hip.hipEventDestroy(e0)
    hip.hipEventDestroy(e1)
    assert torch.equal(out, out0) and torch.equal(lse, lse0)
