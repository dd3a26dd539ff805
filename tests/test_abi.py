"""The C-ABI library loads, exports what include/xattn.h declares, and rejects
bad arguments before enqueuing anything (no GPU needed, no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

from generative_recommendation_beam_xattn_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xattn.h")


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\S.*?\b(xattn_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\b(xattn_\w+)\b", out))
    assert set(names) <= exported


@pytest.mark.parametrize("lang", ["c", "c++"])
def test_header_is_plain_c_and_cxx(lang, tmp_path):
    src = tmp_path / ("t." + ("c" if lang == "c" else "cpp"))
    src.write_text('#include "xattn.h"\nint main(void){xattn_shape s; (void)s; return 0;}\n')
    cc = "gcc" if lang == "c" else "g++"
    subprocess.run([cc, "-fsyntax-only", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                    str(src)], check=True)


def test_status_strings(lib):
    for code, text in [(0, "ok"), (1, "invalid argument"), (2, "unsupported shape or dtype"),
                       (3, "HIP runtime error")]:
        assert lib.xattn_status_string(code).decode() == text


def shape(**kw):
    base = dict(num_requests=2, beam_width=4, num_q_heads=8, num_kv_heads=2, head_dim=128,
                max_prompt_len=64, max_steps=3, dtype=B.XATTN_BF16, scale=0.0)
    base.update(kw)
    return B.Shape(**base)


def test_workspace_size(lib):
    assert B.workspace_size(shape(), 2) == 0
    s = shape(max_steps=40)
    n = 2 * 40 * 4 * 4
    assert B.workspace_size(s, 39) == (n + 255) // 256 * 256
    assert B.workspace_size(s, 15) == 0
    assert B.workspace_size(s, 16) > 0
    assert lib.xattn_workspace_size(ctypes.byref(shape(num_requests=0)), 0) == ctypes.c_size_t(-1).value
    assert lib.xattn_workspace_size(None, 0) == ctypes.c_size_t(-1).value


BAD_SHAPES = [
    (dict(num_requests=0), 1, "num_requests"),
    (dict(beam_width=0), 1, "beam_width"),
    (dict(num_kv_heads=0), 1, "head counts"),
    (dict(num_q_heads=6, num_kv_heads=4), 1, "multiple"),
    (dict(head_dim=96), 2, "head_dim"),
    (dict(head_dim=0), 1, "head_dim"),
    (dict(max_prompt_len=-1), 1, "max_prompt_len"),
    (dict(max_steps=0), 1, "max_steps"),
    (dict(dtype=7), 1, "dtype"),
    (dict(scale=-1.0), 1, "scale"),
    (dict(scale=float("inf")), 1, "scale"),
    (dict(scale=float("nan")), 1, "scale"),
    (dict(num_requests=1 << 20, beam_width=1 << 20), 1, "2^40"),
]


@pytest.mark.parametrize("kw,status,msg", BAD_SHAPES)
def test_bad_shapes_rejected_before_launch(lib, kw, status, msg):
    # every pointer is NULL as well, so nothing could be launched even if a
    # shape check were missing
    s = shape(**kw)
    st = lib.xattn_decode(ctypes.byref(s), *([None] * 7), 0, None, None, 0, None)
    assert st == status
    assert msg in lib.xattn_last_error().decode()
    st = lib.xattn_resolve_ancestors(ctypes.byref(s), None, 0, None, None)
    assert st == status


def test_bad_step_and_null_pointers_rejected(lib):
    s = shape()
    for step in (-1, 3):
        assert lib.xattn_decode(ctypes.byref(s), *([None] * 7), step, None, None, 0, None) == 1
        assert "step" in lib.xattn_last_error().decode()
    assert lib.xattn_decode(ctypes.byref(s), *([None] * 7), 0, None, None, 0, None) == 1
    assert "NULL" in lib.xattn_last_error().decode()
    assert lib.xattn_decode(None, *([None] * 7), 0, None, None, 0, None) == 1


def test_timed_entry_requires_both_events(lib):
    s = shape()
    fake = ctypes.c_void_p(0x1000)
    for start, stop in ((None, fake), (fake, None), (None, None)):
        st = lib.xattn_decode_timed(ctypes.byref(s), *([None] * 7), 0, None, None, 0, None,
                                    start, stop)
        assert st == 1 and "event" in lib.xattn_last_error().decode()


needs_no_gpu = pytest.mark.skipif(
    os.environ.get("HIP_VISIBLE_DEVICES", "") != "-1" and
    __import__("torch").cuda.is_available(),
    reason="uses fake device addresses; run only where no GPU is reachable")


@needs_no_gpu
def test_alignment_and_workspace_checks(lib):
    s = shape(max_steps=40)
    good = [ctypes.c_void_p(0x10000 * (i + 1)) for i in range(8)]
    q, sk, sv, pl, uk, uv, par, out = good
    # misaligned vector operand
    st = lib.xattn_decode(ctypes.byref(s), ctypes.c_void_p(0x10008), sk, sv, pl, uk, uv, par, 39,
                          out, ctypes.c_void_p(0x100000), 1 << 20, None)
    assert st == 1 and "16-byte" in lib.xattn_last_error().decode()
    # deep chain without workspace
    st = lib.xattn_decode(ctypes.byref(s), q, sk, sv, pl, uk, uv, par, 39, out, None, 0, None)
    assert st == 1 and "workspace" in lib.xattn_last_error().decode()
    # workspace too small
    st = lib.xattn_decode(ctypes.byref(s), q, sk, sv, pl, uk, uv, par, 39, out,
                          ctypes.c_void_p(0x100000), 16, None)
    assert st == 1 and "smaller" in lib.xattn_last_error().decode()
    # misaligned workspace
    st = lib.xattn_decode(ctypes.byref(s), q, sk, sv, pl, uk, uv, par, 39, out,
                          ctypes.c_void_p(0x100010), 1 << 20, None)
    assert st == 1 and "256-byte" in lib.xattn_last_error().decode()
    # NULL shared cache with a non-empty capacity
    st = lib.xattn_decode(ctypes.byref(shape()), q, None, None, pl, uk, uv, par, 0, out, None, 0,
                          None)
    assert st == 1 and "shared" in lib.xattn_last_error().decode()
