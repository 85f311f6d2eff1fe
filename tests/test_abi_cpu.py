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


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wts_[a-z_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    from serial_draft_head_persistent_amd import _abi
    assert set(_declared_functions()) == set(_abi.EXPORTS)


def test_library_exports_every_declared_symbol():
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True, text=True).stdout
    for name in _declared_functions():
        assert re.search(rf"\bT {name}$", out, flags=re.M), name


def test_status_strings():
    from serial_draft_head_persistent_amd import _abi
    lib = _abi.load()
    for code in range(7):
        assert lib.wts_status_string(code)
    assert lib.wts_status_string(99) == b"unknown status"


@pytest.mark.parametrize("cname,pyname", [("wts_create_params", "CreateParams"),
                                          ("wts_walk_params", "WalkParams"), ("wts_plan", "Plan")])
def test_struct_layout_matches_c(cname, pyname):
    from serial_draft_head_persistent_amd import _abi
    st = getattr(_abi, pyname)
    fields = [f for f, _ in st._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', '#include "wts.h"', 'int main(void) {',
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
