"""The C-ABI library loads on a machine without a GPU and exports every
symbol include/specverify.h declares (no compute call is made here)."""

import ctypes
import os
import re

import pytest

import target_verification_amd as tva

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "specverify.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_ ]*[\s\*]+([a-z_0-9]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_binding_surface():
    assert set(declared_functions()) == set(tva.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = tva.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_strings_and_version():
    assert tva.sv_version() == 1
    assert tva.sv_status_string(tva.SV_OK) == "ok"
    assert tva.sv_status_string(tva.SV_E_CAPACITY) == "KV capacity exceeded"
    assert tva.sv_status_string(tva.SV_E_UNSUPPORTED) == "unsupported"


def test_struct_layout_matches_header_sizes():
    # three int32 blocks + pointers; the ctypes mirror must match the C layout
    assert ctypes.sizeof(tva.SvKV) == 8 + 3 * 8
    assert ctypes.sizeof(tva.SvRound) == 16 + 8 * 8 + 8 + 8
    assert ctypes.sizeof(tva.SvModelDesc) == 14 * 4 + 12 * 8
    # 2 int32, 5 pointers, int32 + padding, 4 pointers, int32 + 2 floats + padding,
    # 2 pointers
    assert ctypes.sizeof(tva.SvAdvanceArgs) == 8 + 5 * 8 + 8 + 4 * 8 + 16 + 2 * 8


def test_null_arguments_fail_closed_without_gpu():
    lib = tva.lib()
    out = ctypes.c_void_p()
    assert lib.sv_model_create(None, ctypes.byref(out)) == tva.SV_E_INVALID
    assert lib.sv_qweight_create(tva.SV_B4_256, 32, 256, None, ctypes.byref(out)) == \
        tva.SV_E_INVALID
    assert lib.sv_qweight_create(9, 32, 256, ctypes.c_void_p(16), ctypes.byref(out)) == \
        tva.SV_E_UNSUPPORTED
    assert lib.spec_verify_round(None, None, None, None, 0, None) == tva.SV_E_INVALID
    assert lib.spec_verify_round_static(None, None, None, None) == tva.SV_E_INVALID
    assert lib.sv_workspace_bytes(None, 1, 3, 0) == 0
    assert lib.sv_advance(None, None) == tva.SV_E_INVALID
    a = tva.SvAdvanceArgs()
    a.n_seq, a.nt = 1, 3                 # pointers left NULL
    assert lib.sv_advance(ctypes.byref(a), None) == tva.SV_E_INVALID


def test_binding_structs_match_the_c_layout(tmp_path):
    """The ctypes mirrors of the header's structs have the C compiler's
    size and field offsets (the header built as C99 with -pedantic)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    pairs = [("sv_model_desc", tva.SvModelDesc), ("sv_kv", tva.SvKV), ("sv_round", tva.SvRound),
             ("sv_advance_args", tva.SvAdvanceArgs), ("sv_profile_stat", tva.SvProfileStat)]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "specverify.h"',
             'int main(void) {']
    for cname, py in pairs:
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in py._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror",
                    "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(l.split()[:2]): int(l.split()[2]) for l in out if l.strip()}
    for cname, py in pairs:
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for f, _ in py._fields_:
            assert got[(cname, f)] == getattr(py, f).offset, (cname, f)
