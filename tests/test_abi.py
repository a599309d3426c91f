"""The C-ABI library loads and exports every entry point include/iskv.h declares (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "iskv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "return", "sizeof")))


def test_header_declares_the_five_hot_path_calls():
    names = declared_functions()
    for n in ("isvd_init", "isvd_merge_block", "isvd_reorth", "kv_reconstruct", "decode_attend"):
        assert n in names


def test_library_exports_every_declared_symbol():
    import online_rank_kv_amd as K
    lib = ctypes.CDLL(K.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(K.EXPORTED_SYMBOLS) == declared_functions()


def test_host_only_calls():
    import online_rank_kv_amd as K
    cfg = K.IskvConfig(1024, 256, 32, 18432, 256, 0.0, 0)
    ws = K.isvd_workspace_bytes(cfg)
    assert ws > 0
    assert K.isvd_workspace_bytes(K.IskvConfig(1000, 256, 32, 100, 0, 0.0, 0)) == 0  # D % 64
    assert K.isvd_workspace_bytes(K.IskvConfig(1024, 256, 65, 100, 0, 0.0, 0)) == 0  # b_max > 64
    assert K.iskv_strerror(-2) == "capacity exceeded"
    assert K.iskv_window_rows(10, 128, 32) == 170
    assert K.decode_attend_workspace_bytes(1, 1024, 32, 128) > 0
    assert K.decode_attend_workspace_bytes(1, 1024, 32, 64) == 0
    # the batched reconstruction refuses missing arrays and counts outside
    # 1 .. 32 before touching any handle or device memory
    lib = K.lib
    assert lib.kv_reconstruct_batched(None, 1, None, None, None, 128, 5e5, None) == -1
    hs = (ctypes.c_void_p * 1)(None)
    outs = (ctypes.c_void_p * 1)(None)
    nt = (ctypes.c_int32 * 1)(0)
    rp = (ctypes.c_int32 * 1)(0)
    assert lib.kv_reconstruct_batched(hs, 0, outs, nt, rp, 128, 5e5, None) == -1
    assert lib.kv_reconstruct_batched(hs, 33, outs, nt, rp, 128, 5e5, None) == -1
    assert lib.kv_reconstruct_batched(hs, 1, outs, nt, rp, 128, 5e5, None) == -1  # null handle


def test_no_cpu_fallback_in_product_package():
    """The product package never imports the oracle (it must fail loudly without the HIP library)."""
    pkg = os.path.join(ROOT, "online_rank_kv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in src and "from oracle" not in src, f
