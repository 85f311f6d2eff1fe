"""CPU checks of the C ABI: the library loads, exports every function that
include/wts.h declares, and the ctypes structures match the C layout."""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wts.h")
ROOFLINE_HEADER = os.path.join(ROOT, "include", "wts_roofline.h")


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wts_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    from serial_draft_head_persistent_amd import _abi
    assert set(_declared_functions()) == set(_abi.EXPORTS)


def test_roofline_header_declares_its_entry_point():
    from serial_draft_head_persistent_amd import _abi
    assert set(_declared_functions(ROOFLINE_HEADER)) == set(_abi.ROOFLINE_EXPORTS)


def test_library_exports_every_declared_symbol():
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    names = _declared_functions() + _declared_functions(ROOFLINE_HEADER)
    for name in names:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True).stdout
    for name in names:
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings():
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    for code in range(7):
        assert lib.wts_status_string(code)
    assert lib.wts_status_string(99) == b"unknown status"


@pytest.mark.parametrize("cname,pyname", [("wts_create_params", "CreateParams"),
                                          ("wts_walk_params", "WalkParams"), ("wts_plan", "Plan"),
                                          ("wts_roofline_result", "RooflineResult")])
def test_struct_layout_matches_c(cname, pyname):
    from serial_draft_head_persistent_amd import _abi
    st = getattr(_abi, pyname)
    fields = [f for f, _ in st._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "wts.h"', '#include "wts_roofline.h"',
           'int main(void) {',
           f'  printf("%zu\\n", sizeof({cname}));']
    src += [f'  printf("%zu\\n", offsetof({cname}, {f}));' for f in fields]
    src += ['  return 0;', '}']
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write("\n".join(src))
        exe = os.path.join(d, "t")
        subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(st)
    for f, off in zip(fields, vals[1:]):
        assert getattr(st, f).offset == off, f


def _valid_create_params(_abi):
    # fake, 256-byte aligned, never dereferenced: every case below is rejected
    # before the library touches a device
    fake = 0x7F0000000000
    return _abi.CreateParams(V=4096, r=256, head=0, wtype=0, W=fake, w_scale=fake, E=fake, A=None, c=None,
                             max_batch=16, max_steps=64, resident_tiles=-1, lds_tiles=-1, device=0,
                             cooperative=0, watchdog_us=0)


@pytest.mark.parametrize("field,value,status", [
    ("V", 0, 1), ("V", 262144, 1), ("r", 0, 1), ("r", 128, 2), ("head", 2, 1), ("wtype", 2, 1),
    ("W", None, 1), ("E", None, 1), ("w_scale", None, 1), ("max_batch", 0, 1), ("max_batch", 17, 1),
    ("max_steps", 0, 1), ("max_steps", 65, 1), ("resident_tiles", -2, 1), ("lds_tiles", -2, 1),
    ("W", 0x7F0000000008, 1), ("E", 0x7F0000000004, 1), ("grid", -1, 1), ("grid", 257, 1),
    ("exchange", 2, 1), ("exchange", -1, 1),
])
def test_create_rejects_bad_arguments_before_any_device_call(field, value, status):
    """Host-detectable errors of wts_create return a status (1 = invalid
    argument, 2 = unsupported) and leave *out NULL."""
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    p = _valid_create_params(_abi)
    setattr(p, field, value)
    h = ctypes.c_void_p(0x1234)
    assert lib.wts_create(ctypes.byref(p), ctypes.byref(h)) == status
    assert not h.value


def test_recurrent_create_needs_A_and_c():
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    p = _valid_create_params(_abi)
    p.head = 1
    h = ctypes.c_void_p()
    assert lib.wts_create(ctypes.byref(p), ctypes.byref(h)) == 1
    p.A = 0x7F0000000000
    assert lib.wts_create(ctypes.byref(p), ctypes.byref(h)) == 1  # c still missing
    assert not h.value


def test_null_context_and_params_are_rejected():
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    h = ctypes.c_void_p()
    assert lib.wts_create(None, ctypes.byref(h)) == 1
    p = _valid_create_params(_abi)
    assert lib.wts_create(ctypes.byref(p), None) == 1
    w = _abi.WalkParams(B=1, gamma=1)
    assert lib.wts_walk(None, ctypes.byref(w)) == 1
    plan = _abi.Plan()
    assert lib.wts_get_plan(None, 1, 0, 0, ctypes.byref(plan)) == 1
    lib.wts_destroy(None)  # a no-op
    assert lib.wts_roofline(0, None) == 1
    r = _abi.RooflineResult()
    assert lib.wts_roofline(-1, ctypes.byref(r)) == 1
