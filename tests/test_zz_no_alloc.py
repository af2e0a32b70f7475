"""The no-allocation entry point (kv4_append_decode_attention_noalloc) against
kv4_append_decode_attention with a caller workspace, on copies of the same
cache: pages, side rows, out and lse bit-identical.  Two calls in a row share
the library's fixed scratch, the second with a smaller batch; then a batch
beyond the 256-sequence register plan (the plan kernel writes into the
scratch too), and a batch too large for the scratch, refused on the host."""
import ctypes

import numpy as np
import pytest
import torch

import int8_mixed_precision_kv4_amd as kv4
from synth import make_workload
from tests.gpu_util import SCALE, bf, i32
from tests.wl import host_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _say(msg):
    print(msg, flush=True)


def _prefilled(wl, hi, dev):
    """Cache holding positions [0, ctx-1) of every sequence (re-prefill)."""
    cache = kv4.Kv4Cache.zeros(wl.num_pages, wl.Hkv, wl.max_slots, dev)
    lead = wl.ctx - 1
    k, v, cu = hi.prefix(lead)
    if len(k):
        kv4.prefill_quantize(cache, bf(k, dev), bf(v, dev), i32(cu, dev), i32(np.zeros(wl.B), dev),
                             i32(wl.slots, dev), i32(wl.page_table, dev), int(max(1, lead.max())))
    return cache


def _clone(c):
    return kv4.Kv4Cache(c.pages.clone(), c.side_codes.clone(), c.side_scales.clone(), c.sink, c.window)


def _compare(wl, dev, label):
    hi = host_inputs(wl)
    base = _prefilled(wl, hi, dev)
    table, slots = i32(wl.page_table, dev), i32(wl.slots, dev)
    ka, va = hi.at(wl.ctx - 1)
    k_new, v_new, pos = bf(ka, dev), bf(va, dev), i32(wl.ctx - 1, dev)
    q, ctx = bf(hi.q, dev), i32(wl.ctx, dev)
    a, b = _clone(base), _clone(base)
    o1, l1 = kv4.append_decode_attention(a, k_new, v_new, pos, q, ctx, slots, table, wl.max_ctx, SCALE)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    kv4.append_decode_attention_noalloc(b, k_new, v_new, pos, q, ctx, slots, table, wl.max_ctx, SCALE, o2, l2)
    torch.cuda.synchronize()
    _say(f"[noalloc] {label}: B={wl.B} Hq/Hkv={wl.Hq}/{wl.Hkv} max ctx {wl.max_ctx} compared")
    assert torch.equal(a.pages, b.pages), label
    assert torch.equal(a.side_codes, b.side_codes) and torch.equal(a.side_scales, b.side_scales), label
    assert torch.equal(o1, o2), label
    assert torch.equal(l1, l2), label


def test_noalloc_equals_workspace_call_twice_then_smaller():
    dev = torch.device("cuda")
    _compare(make_workload(1), dev, "first call (short workload, 64 sequences)")
    _compare(make_workload(0), dev, "second call, smaller (tiny workload, 4 sequences)")


def test_noalloc_plan_kernel_batch():
    """300 sequences of short and edge contexts: the plan kernel's prefix sums
    live in the scratch as well."""
    dev = torch.device("cuda")
    rng = np.random.default_rng(11)
    ctx = rng.choice([1, 2, 16, 17, 143, 144, 145, 160, 200, 333, 700], size=300)
    _compare(make_workload(0, ctx=ctx, Hq=8, Hkv=2, seed=121), dev, "plan-kernel batch (300 sequences)")


def test_noalloc_refuses_a_batch_beyond_the_scratch():
    """65535 sequences x 32 q-heads need far more than the fixed scratch: the
    call returns KV4_ERR_WORKSPACE on the host, before anything is enqueued
    (the tiny buffers passed here are never read)."""
    dev = torch.device("cuda")
    cache = kv4.Kv4Cache.zeros(4, 8, 1, dev)
    small = torch.zeros(64, dtype=torch.int32, device=dev)
    need = kv4.decode_workspace_bytes(cache, 65535, 32, 16)
    assert need > kv4.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(small.data_ptr())
    rc = kv4.lib().kv4_append_decode_attention_noalloc(cache.desc(), p, p, p, p, p, p, p, 1, 65535, 32, 16,
                                                       SCALE, p, p, None)
    assert rc == -4
    torch.cuda.synchronize()
