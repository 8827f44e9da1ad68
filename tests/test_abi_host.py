"""The C ABI on the host (no GPU needed): the library loads, exports every
entry point include/fs.h declares, its struct layout and constants agree with
the Python binding, and host-checkable errors are returned before any HIP
call (so they work on a machine without a GPU)."""

import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fs.h")

fs = pytest.importorskip("kv_cache_injection_amd.fs",
                         reason="libfs.so not built (run __graft_entry__.build())")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"FS_API\s+[\w\s\*]+?\b(fs_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(fs.EXPORTS)
    lib = ctypes.CDLL(fs.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", fs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == names


def test_constants_match_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define\s+(FS_\w+)\s+\(?(-?(?:0x)?[0-9a-fA-F]+)u?\)?", text))
    checked = 0
    for name, val in defs.items():
        if hasattr(fs, name):
            assert getattr(fs, name) == int(val, 0), name
            checked += 1
    assert checked == 22


def test_desc_layout_matches_c(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "fs.h"\n'
                   "int main(void){printf(\"%zu\", sizeof(fs_store_desc));"
                   + "".join(f'printf(" %zu", offsetof(fs_store_desc, {f}));'
                             for f, _ in fs.fs_store_desc._fields_)
                   + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    vals = list(map(int, subprocess.run([str(exe)], capture_output=True, text=True,
                                        check=True).stdout.split()))
    assert vals[0] == ctypes.sizeof(fs.fs_store_desc)
    assert vals[1:] == [getattr(fs.fs_store_desc, f).offset for f, _ in fs.fs_store_desc._fields_]


def test_strerror():
    for code in range(8):
        assert fs.fs_strerror(code)
    assert fs.fs_strerror(0) == "ok"
    assert "unknown" in fs.fs_strerror(99)


def _good_desc():
    return fs.make_desc(num_layers=2, num_kv_heads=8, head_dim=128, embed_dim=384,
                        rope_theta=5e5, block_size=16, num_users=2, max_batch=4, max_k=8,
                        num_facts=4, num_tokens=40)


FAKE = 0x10000   # aligned, never dereferenced: every case below fails validation first


def _create(desc, ufb=(0, 2, 4), fl=(10, 10, 10, 10), emb=FAKE, arenas=None):
    ufb = np.asarray(ufb, np.int64)
    fl = np.asarray(fl, np.int32)
    n = desc.num_layers if desc.num_layers > 0 else 1
    arenas = arenas if arenas is not None else [FAKE] * n
    arr = (ctypes.c_void_p * len(arenas))(*arenas)
    out = ctypes.c_void_p(0)
    st = fs._lib.fs_create_store(ctypes.byref(desc), ufb.ctypes.data_as(ctypes.c_void_p),
                                 fl.ctypes.data_as(ctypes.c_void_p), ctypes.c_void_p(emb),
                                 arr, arr, None, ctypes.byref(out))
    return st, out


@pytest.mark.parametrize("field, value, status", [
    ("num_layers", 0, fs.FS_E_ARG),
    ("num_layers", 129, fs.FS_E_ARG),
    ("num_kv_heads", 0, fs.FS_E_ARG),
    ("num_kv_heads", 65, fs.FS_E_UNSUPPORTED),     # 65 x 128: rows above 16 KB
    ("head_dim", 100, fs.FS_E_ARG),
    ("head_dim", 96, fs.FS_E_UNSUPPORTED),
    ("embed_dim", 6, fs.FS_E_ARG),
    ("embed_dim", 8192, fs.FS_E_UNSUPPORTED),
    ("rope_theta", 1.0, fs.FS_E_ARG),
    ("rope_theta", float("inf"), fs.FS_E_ARG),
    ("block_size", 12, fs.FS_E_ARG),
    ("block_size", 2048, fs.FS_E_ARG),
    ("kv_location", 5, fs.FS_E_ARG),
    ("num_users", 0, fs.FS_E_ARG),
    ("max_batch", 0, fs.FS_E_ARG),
    ("max_k", 0, fs.FS_E_ARG),
    ("max_k", 1025, fs.FS_E_ARG),
    ("num_facts", 0, fs.FS_E_ARG),
    ("num_tokens", 0, fs.FS_E_ARG),
])
def test_create_rejects_bad_desc(field, value, status):
    d = _good_desc()
    setattr(d, field, value)
    st, out = _create(d)
    assert st == status
    assert out.value is None
    assert fs.fs_last_error_message()


def test_create_rejects_pinned_without_staging():
    d = _good_desc()
    d.kv_location = fs.FS_KV_PINNED_HOST
    d.staging_layers = 0
    assert _create(d)[0] == fs.FS_E_ARG
    d.staging_layers = 3
    assert _create(d)[0] == fs.FS_E_ARG


@pytest.mark.parametrize("kw", [
    dict(ufb=(1, 2, 4)),                 # must start at 0
    dict(ufb=(0, 3, 2)),                 # decreasing
    dict(ufb=(0, 2, 3)),                 # does not end at num_facts
    dict(fl=(10, 10, 0, 20)),            # empty fact
    dict(fl=(10, 10, 10, 11)),           # lengths exceed num_tokens
    dict(emb=FAKE + 4),                  # misaligned embeddings
    dict(arenas=[FAKE, FAKE + 8]),       # misaligned arena
    dict(arenas=[FAKE, 0]),              # null arena
])
def test_create_rejects_bad_metadata(kw):
    st, out = _create(_good_desc(), **kw)
    assert st == fs.FS_E_ARG
    assert out.value is None


def test_null_store_is_rejected_everywhere():
    L = fs._lib
    flags = ctypes.c_uint32()
    assert L.fs_retrieve_topk(None, 1, FAKE, FAKE, 1, FAKE, None, None, None) == fs.FS_E_ARG
    arr = (ctypes.c_void_p * 1)(FAKE)
    assert L.fs_inject(None, 0, 1, FAKE, FAKE, 1, FAKE, 4, FAKE, arr, arr, 4, None) == fs.FS_E_ARG
    assert L.fs_inject_layers(None, 0, 1, 1, FAKE, FAKE, 1, FAKE, 4, FAKE, arr, arr, 4, None) == fs.FS_E_ARG
    assert L.fs_fetch_async(None, 1, FAKE, FAKE, 1, 0, 1, None) == fs.FS_E_ARG
    n = ctypes.c_size_t()
    assert L.fs_inject_plan_size(None, 1, ctypes.byref(n)) == fs.FS_E_ARG
    assert L.fs_plan_inject(None, 1, FAKE, FAKE, 1, FAKE, 4, FAKE, 4, FAKE, 1 << 20, None) == fs.FS_E_ARG
    assert L.fs_inject_planned(None, 0, 1, 1, 1, FAKE, 1 << 20, arr, arr, 4, None) == fs.FS_E_ARG
    assert L.fs_inject_noalloc(None, 0, 1, FAKE, FAKE, 1, FAKE, 1, FAKE, arr, arr, 4, None) == fs.FS_E_ARG
    assert L.fs_retrieve_plan(None, 1, FAKE, FAKE, 1, FAKE, None, None, FAKE, 4, FAKE, 4, FAKE, 1 << 20,
                              None) == fs.FS_E_ARG
    assert L.fs_poll_errors(None, None, ctypes.byref(flags)) == fs.FS_E_ARG
    assert L.fs_destroy_store(None) == fs.FS_OK
