"""The C-ABI library loads and exports every function include/kv4.h declares
(no GPU needed: nothing is called)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kv4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(kv[48][a-z0-9_]*)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("kv4_append", "kv4_prefill_quantize", "kv4_decode_attention",
                     "kv4_decode_workspace_bytes", "kv4_strerror", "kv4bench_bf16_paged_decode"):
        assert required in names


def test_library_exports_every_declared_symbol():
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(kv4.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(kv4.EXPORTS)


def test_strerror_without_gpu():
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built")
    L = kv4.lib()
    assert L.kv4_strerror(0) == b"success"
    assert b"workspace" in L.kv4_strerror(-4)


def test_host_validation_rejects_bad_arguments_without_gpu():
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built")
    L = kv4.lib()
    # NULL descriptor and unsupported geometry are refused before any HIP call
    assert L.kv4_append(None, None, None, None, None, None, 1, 1, None) == -1
    d = kv4._Desc(1, 4, 32, 1, 128, 16, 128, 1, 1, 1, 1)  # page_size 32
    assert L.kv4_append(ctypes.byref(d), 1, 1, 1, None, 1, 1, 1, None) == -2
    d = kv4._Desc(1, 4, 16, 1, 128, 16, 128, 1, 1, 1, 1)
    assert L.kv4_append(ctypes.byref(d), 1, 1, 1, None, 1, 1, 0, None) == -3


@pytest.mark.parametrize("sink,window,ok", [
    (16, 128, True), (0, 0, True), (144, 0, True), (0, 144, True), (32, 64, True),
    (8, 0, False), (16, 129, False), (-16, 0, False), (0, -1, False), (160, 0, False)])
def test_host_validation_of_the_protection_budget(sink, window, ok):
    """A budget is accepted when s is a non-negative multiple of 16, w >= 0 and
    s + w <= 144 (then a NULL k is what fails); otherwise refused as
    unsupported before any HIP call."""
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built")
    L = kv4.lib()
    d = kv4._Desc(1, 4, 16, 1, 128, sink, window, 1, 1, 1, 1)
    want = -1 if ok else -2
    assert L.kv4_append(ctypes.byref(d), None, 1, 1, None, 1, 1, 1, None) == want
    assert L.kv4_prefill_quantize(ctypes.byref(d), None, 1, 1, 1, None, 1, 1, 1, 1, None) == want
    assert L.kv4_decode_attention(ctypes.byref(d), None, 1, None, 1, 1, 1, 4, 16, 1.0, 1, 1, 1, 1,
                                  None) == want


def test_noalloc_entry_point_refuses_beyond_its_scratch_without_gpu():
    """kv4_append_decode_attention_noalloc: a batch whose workspace exceeds the
    fixed scratch is refused with KV4_ERR_WORKSPACE before any launch (the
    pointers are dummies and never touched); NULL inputs give KV4_ERR_NULLPTR."""
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built")
    L = kv4.lib()
    d = kv4._Desc(1, 4, 16, 8, 128, 16, 128, 1, 1, 1, 1)
    big = L.kv4_decode_workspace_bytes(ctypes.byref(d), 65535, 32, 16)
    assert big > kv4.NOALLOC_SCRATCH_BYTES
    assert L.kv4_append_decode_attention_noalloc(ctypes.byref(d), 1, 1, 1, 1, 1, 1, 1, 1, 65535, 32, 16,
                                                 0.1, 1, 1, None) == -4
    assert L.kv4_append_decode_attention_noalloc(ctypes.byref(d), None, 1, 1, 1, 1, 1, 1, 1, 4, 32, 16,
                                                 0.1, 1, 1, None) == -1
    # the benchmark's batch (256 sequences, 32/8 heads) fits with room to spare
    assert L.kv4_decode_workspace_bytes(ctypes.byref(d), 256, 32, 16384) <= kv4.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("Hq,Hkv", [(6, 4), (5, 2), (12, 8), (3, 4), (0, 8), (-8, 8)])
def test_query_heads_not_a_multiple_of_kv_heads_are_refused_without_gpu(Hq, Hkv):
    """Every query head reads one kv-head, so Hq must be a positive multiple of
    Hkv; anything else is refused as unsupported on the host, before any
    launch, by every decode-side entry point (the pointers are dummies and
    never touched), and its workspace size is 0."""
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built")
    L = kv4.lib()
    d = kv4._Desc(1, 4, 16, Hkv, 128, 16, 128, 1, 1, 1, 1)
    assert L.kv4_decode_attention(ctypes.byref(d), 1, 1, None, 1, 1, 1, Hq, 16, 1.0, 1, 1, 1, 1 << 30,
                                  None) == -2
    assert L.kv4_append_decode_attention(ctypes.byref(d), 1, 1, 1, 1, 1, None, 1, 1, 1, Hq, 16, 1.0, 1, 1,
                                         1, 1 << 30, None) == -2
    assert L.kv4_append_decode_attention_noalloc(ctypes.byref(d), 1, 1, 1, 1, 1, None, 1, 1, 1, Hq, 16,
                                                 1.0, 1, 1, None) == -2
    assert L.kv4_prefill_attention(ctypes.byref(d), 1, 1, 1, None, 1, 1, 1, 1, Hq, 16, 1.0, 1, 1, 1,
                                   1 << 30, None) == -2
    assert L.kv4mx_decode_attention(ctypes.byref(d), 1, 1, None, 1, 1, 1, Hq, 16, 1.0, 1, 1, 1, 1 << 30,
                                    None) == -2
    assert L.kv4_decode_workspace_bytes(ctypes.byref(d), 4, Hq, 64) == 0
    assert L.kv4_prefill_attention_workspace_bytes(ctypes.byref(d), 4, Hq, 64) == 0
    d8 = kv4._Kv8Desc(1, 4, 16, Hkv, 128, 1)
    assert L.kv8_decode_attention(ctypes.byref(d8), 1, 1, 1, 1, 1, Hq, 16, 1.0, 1, 1, 1, 1 << 30, None) == -2
    assert L.kv8_decode_workspace_bytes(ctypes.byref(d8), 4, Hq, 64) == 0
    assert L.kv4bench_bf16_paged_decode(1, 4, Hkv, 1, 1, 1, 1, 1, Hq, 16, 1.0, 1, 1, 1, 1 << 30, None) == -2


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (16, 2), (64, 8), (6, 2), (5, 1)])
def test_group_sizes_other_than_four_take_more_groups_without_gpu(Hq, Hkv):
    """Any whole group size G = Hq/Hkv is taken: the kernels' rows are virtual
    groups of at most 4 query heads of one kv-head, ceil(G/4) of them per
    kv-head, each with its own chunk partials. Only the BF16 comparator keeps
    G = 4."""
    import int8_mixed_precision_kv4_amd as kv4
    if not os.path.exists(kv4.LIB_PATH):
        pytest.skip("libkv4.so not built")
    L = kv4.lib()
    d = kv4._Desc(1, 4, 16, Hkv, 128, 16, 128, 1, 1, 1, 1)
    ws = L.kv4_decode_workspace_bytes(ctypes.byref(d), 4, Hq, 64)
    assert ws > 0
    # four more query heads per kv-head add one group per kv-head: more partials
    assert L.kv4_decode_workspace_bytes(ctypes.byref(d), 4, Hq + 4 * Hkv, 64) > ws
    assert L.kv4_prefill_attention_workspace_bytes(ctypes.byref(d), 4, Hq, 64) > 0
    d8 = kv4._Kv8Desc(1, 4, 16, Hkv, 128, 1)
    assert L.kv8_decode_workspace_bytes(ctypes.byref(d8), 4, Hq, 64) > 0
    assert L.kv4bench_bf16_paged_decode(1, 4, Hkv, 1, 1, 1, 1, 1, Hq, 16, 1.0, 1, 1, 1, 1 << 30, None) == -2


def test_binding_checks_dtypes_and_shapes_without_gpu():
    """The Python binding refuses, on the host, arguments whose element type
    or leading dimension the library would misread on the device."""
    import torch

    import int8_mixed_precision_kv4_amd as kv4
    cache = kv4.Kv4Cache.zeros(4, 1, 2, device="cpu")
    B = 2
    q = torch.zeros((B, 4, 128), dtype=torch.bfloat16)
    ctx = torch.ones(B, dtype=torch.int32)
    table = torch.zeros((B, 1), dtype=torch.int32)
    bad = [dict(q=q.float()), dict(ctx_len=ctx.long()), dict(page_table=table.long()),
           dict(ctx_len=torch.ones(B + 1, dtype=torch.int32)), dict(page_table=table[:1]),
           dict(slot=torch.zeros(B, dtype=torch.int64))]
    for change in bad:
        args = dict(q=q, ctx_len=ctx, slot=None, page_table=table)
        args.update(change)
        with pytest.raises(kv4.Kv4Error):
            kv4.decode_attention(cache, args["q"], args["ctx_len"], args["slot"], args["page_table"], 16, 0.1)
    with pytest.raises(kv4.Kv4Error):  # int64 positions for an append
        kv4.append(cache, q[:, :1].contiguous(), q[:, :1].contiguous(), torch.zeros(B, dtype=torch.int64), None,
                   table)
    with pytest.raises(kv4.Kv4Error):  # float32 keys for a re-prefill
        kv4.prefill_quantize(cache, torch.zeros((3, 1, 128)), torch.zeros((3, 1, 128)),
                             torch.tensor([0, 3], dtype=torch.int32), torch.zeros(1, dtype=torch.int32), None,
                             table[:1], 3)
