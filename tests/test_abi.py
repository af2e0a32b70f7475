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
