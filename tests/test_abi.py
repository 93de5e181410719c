"""The C-ABI library loads, exports every symbol its headers declare, and its
validation rejects bad arguments before touching a GPU (no GPU needed)."""
import ctypes
import glob
import os
import re

import pytest

from mxfp4_routed_expert_renorm_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*[A-Za-z_][\w\s\*]*?\b(moe_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("library not built: run __graft_entry__.build()")
    return B.load()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in sorted(names):
        assert hasattr(lib, n), n


def _struct_fields(name):
    """Field names of a typedef'd struct in the headers, in declaration order."""
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        m = re.search(r"typedef struct\s*\{([^}]*)\}\s*" + name + r"\s*;", src)
        if m:
            fields = []
            for decl in m.group(1).split(";"):
                decl = decl.strip()
                if decl:
                    head, *rest = decl.split(",")
                    fields.append(re.findall(r"(\w+)\s*$", head)[0])
                    fields += [r.strip().lstrip("*").strip() for r in rest]
            return fields
    raise AssertionError(name)


@pytest.mark.parametrize("cname,pyname", [("moe_layer", "moe_layer"), ("moe_cache_desc", "moe_cache_desc"),
                                          ("moe_cache_stats", "moe_cache_stats")])
def test_binding_structs_match_header(cname, pyname):
    assert [f for f, _ in getattr(B, pyname)._fields_] == _struct_fields(cname)


def test_sizes_match_pages(lib):
    assert lib.moe_fp4_expert_bytes(4096, 2048) == 13369344
    assert lib.moe_int2_expert_bytes(4096, 2048) == 7077888
    assert lib.moe_fp4_expert_bytes(0, 2048) == 0


def _status(lib, fn, *args):
    st = getattr(lib, fn)(*args)
    return st, lib.moe_last_error().decode()


FAKE = ctypes.c_void_p(0x1000)


def test_route_validation(lib):
    st, msg = _status(lib, "moe_route", FAKE, 1, 8, 9, FAKE, FAKE, None)
    assert st == 1 and "k=9" in msg
    st, msg = _status(lib, "moe_route", FAKE, 1, 2000, 8, FAKE, FAKE, None)
    assert st == 2 and "E=2000" in msg
    st, msg = _status(lib, "moe_route", None, 4, 8, 2, FAKE, FAKE, None)
    assert st == 1 and "NULL" in msg
    st, msg = _status(lib, "moe_route", FAKE, -1, 8, 2, FAKE, FAKE, None)
    assert st == 2


def test_group_validation(lib):
    st, msg = _status(lib, "moe_group", FAKE, 10, 0, FAKE, FAKE, FAKE, None)
    assert st == 2 and "nkeys" in msg
    st, msg = _status(lib, "moe_group", FAKE, 10, 5000, FAKE, FAKE, FAKE, None)
    assert st == 2


def test_group_wide_validation(lib):
    assert lib.moe_group_scratch_bytes(2048, 257) == 0          # small: the one-workgroup grouping
    assert lib.moe_group_scratch_bytes(36864, 257) == 72 * 257 * 4
    assert lib.moe_group_scratch_bytes(36864, 2000) == 0        # many keys: the one-workgroup grouping
    st, msg = _status(lib, "moe_group_wide", FAKE, 36864, 257, FAKE, FAKE, FAKE, None, None)
    assert st == 1 and "scratch" in msg
    st, msg = _status(lib, "moe_group_wide", FAKE, 36864, 257, FAKE, FAKE, FAKE, 0x1002, None)
    assert st == 1 and "aligned" in msg
    st, msg = _status(lib, "moe_group_wide", FAKE, -1, 257, FAKE, FAKE, FAKE, FAKE, None)
    assert st == 2


def test_expert_forward_validation(lib):
    good = B.moe_layer(256, 128, 0x1000, lib.moe_fp4_expert_bytes(256, 128), 8, None, 0, 0, None)
    ws = lib.moe_expert_workspace_bytes(256, 128, 4, 2, 0)
    args = lambda layer, xt=0, T=4, k=2, w=FAKE, ot=0, wsb=ws: _status(
        lib, "moe_expert_forward", ctypes.byref(layer), FAKE, xt, T, k, FAKE, None, w, FAKE, ot,
        ctypes.c_void_p(0x10000), wsb, None)
    bad_h = B.moe_layer(300, 128, 0x1000, 10 ** 6, 8, None, 0, 0, None)
    st, msg = args(bad_h)
    assert st == 2 and "H=300" in msg
    short = B.moe_layer(256, 128, 0x1000, 100, 8, None, 0, 0, None)
    st, msg = args(short)
    assert st == 1 and "fp4_stride" in msg
    st, msg = args(good, wsb=ws - 1)
    assert st == 4 and "workspace" in msg
    st, msg = args(good, k=0)
    assert st == 1
    st, msg = args(good, xt=7)
    assert st == 1
    st, msg = args(good, w=None, ot=1)
    assert st == 1 and "fp32" in msg
    unaligned = B.moe_layer(256, 128, 0x1001, lib.moe_fp4_expert_bytes(256, 128), 8, None, 0, 0, None)
    st, msg = args(unaligned)
    assert st == 1 and "aligned" in msg
    st, msg = _status(lib, "moe_expert_forward", None, FAKE, 0, 1, 1, FAKE, None, FAKE, FAKE, 0, FAKE, ws, None)
    assert st == 1 and "layer is NULL" in msg


def test_layer_decode_validation(lib):
    rb = lib.moe_fp4_expert_bytes(2048, 2048)
    ws = lib.moe_expert_workspace_bytes(2048, 2048, 1, 8, 0)
    wsp = ctypes.c_void_p(0x10000)
    call = lambda layer, E=64, k=8, xt=1, wsb=ws: _status(
        lib, "moe_layer_decode", ctypes.byref(layer), FAKE, E, FAKE, xt, k, FAKE, FAKE, FAKE, 1, wsp, wsb, None)
    small = B.moe_layer(2048, 2048, 0x1000, rb, 32, None, 0, 0, None)
    st, msg = call(small)
    assert st == 3 and "num_slots=32 < E=64" in msg          # MOE_ECACHE_SMALL
    full = B.moe_layer(2048, 2048, 0x1000, rb, 64, None, 0, 0, None)
    st, msg = call(full, k=65)
    assert st == 1 and "k=65" in msg
    st, msg = call(full, E=2000)
    assert st == 2 and "E=2000" in msg
    st, msg = call(full, wsb=ws - 1)
    assert st == 4 and "workspace" in msg
    st, msg = call(full, xt=9)
    assert st == 1 and "dtype" in msg


def test_layer_decode_noalloc_validation(lib):
    """The allocation-free decode refuses a NULL layer, a bad k and a layer
    whose workspace exceeds the static scratch before it touches a device."""
    call = lambda layer, k=8: _status(lib, "moe_layer_decode_noalloc", layer, FAKE, 256, FAKE, 1, k, FAKE, FAKE,
                                      FAKE, 1, None)
    st, msg = call(None)
    assert st == 1 and "layer is NULL" in msg
    big = B.moe_layer(8192, 8192, 0x1000, lib.moe_fp4_expert_bytes(8192, 8192), 256, None, 0, 0, 0x2000)
    st, msg = call(ctypes.byref(big), k=0)
    assert st == 1 and "k=0" in msg
    st, msg = call(ctypes.byref(big), k=64)
    assert st == 4 and "static scratch" in msg
    assert lib.moe_expert_workspace_sync_offset(8192, 8192, 1, 64, 1) > lib.moe_noalloc_scratch_bytes()


def test_last_error_is_thread_local(lib):
    import threading
    _status(lib, "moe_route", FAKE, 1, 8, 9, FAKE, FAKE, None)
    main_msg = lib.moe_last_error().decode()
    seen = {}

    def other():
        seen["before"] = lib.moe_last_error().decode()
        lib.moe_route(FAKE, 1, 2000, 8, FAKE, FAKE, None)
        seen["after"] = lib.moe_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["before"] == ""
    assert "E=2000" in seen["after"]
    assert lib.moe_last_error().decode() == main_msg


def test_stream_read_validation(lib):
    import ctypes
    n = ctypes.c_size_t
    assert lib.moe_debug_stream_read(None, n(16), None, None) == 1                            # MOE_EINVAL: NULL
    assert lib.moe_debug_stream_read(ctypes.c_void_p(8), n(16), ctypes.c_void_p(64), None) == 1   # misaligned
    assert lib.moe_debug_stream_read(ctypes.c_void_p(64), n(17), ctypes.c_void_p(64), None) == 1  # not a multiple of 16
    assert lib.moe_debug_stream_read(ctypes.c_void_p(64), n(0), ctypes.c_void_p(64), None) == 0   # nothing to read


def test_tp_slice_validation(lib):
    import ctypes
    n = ctypes.c_size_t
    P = ctypes.c_void_p(256)
    # I = 2048 over G = 3 does not divide; G = 128 leaves 16-element slices (not whole scale blocks)
    assert lib.moe_tp_slice(P, n(1 << 24), 1, 4096, 2048, 3, 0, P, n(1 << 24), None) == 2
    assert lib.moe_tp_slice(P, n(1 << 24), 1, 4096, 2048, 128, 0, P, n(1 << 24), None) == 2
    assert lib.moe_tp_slice(P, n(1 << 24), 1, 4096, 2048, 4, 4, P, n(1 << 24), None) == 1   # rank out of range
    assert lib.moe_tp_slice(P, n(16), 1, 4096, 2048, 4, 0, P, n(1 << 24), None) == 1        # stride too small
    assert lib.moe_tp_slice(P, n(1 << 24), 0, 4096, 2048, 4, 0, P, n(1 << 24), None) == 0   # nothing to do
