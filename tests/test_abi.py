"""The C ABI library loads and exports every function include/tod.h declares (no GPU needed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tod.h")
LIB = os.path.join(ROOT, "throughput_oriented_offloaded_amd", "libtod.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|void|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(", text,
                       flags=re.M)
    return sorted(set(names))


def test_header_declares_the_core_calls():
    names = _declared()
    for n in ("init_model", "prefill", "decode_block", "quantize_groupwise"):
        assert n in names
    assert len(names) >= 19


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.fail("libtod.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_header():
    from throughput_oriented_offloaded_amd import _lib
    assert set(_lib.EXPORTED) == set(_declared())


def _struct_fields(name):
    """(field, C type) pairs of `typedef struct { ... } name;` in the header, in order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct\s*\{([^}]*)\}\s*" + name + r"\s*;", text).group(1)
    fields = []
    for decl in body.split(";"):
        decl = decl.strip()
        if decl:
            ctype, names = decl.split(None, 1)
            assert ctype in ("int32_t", "double"), decl
            fields += [(f.strip(), ctype) for f in names.split(",")]
    return fields


@pytest.mark.parametrize("cname,pyname", [("tod_model_config", "ModelConfig"), ("tod_run_config", "RunConfig"),
                                          ("tod_hw", "HW"), ("tod_estimate", "Estimate")])
def test_binding_structs_match_header(cname, pyname):
    """The ctypes mirrors of the header's structs have its fields, in order, with matching types."""
    from throughput_oriented_offloaded_amd import _lib
    py = getattr(_lib, pyname)
    ctypes_of = {"int32_t": ctypes.c_int32, "double": ctypes.c_double}
    assert [(f, t) for f, t in py._fields_] == [(f, ctypes_of[c]) for f, c in _struct_fields(cname)]


def test_library_exports_only_the_declared_functions():
    """Built with hidden visibility: the exported functions are exactly the header's."""
    import shutil
    import subprocess
    if not shutil.which("nm"):
        pytest.skip("nm is not available")
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = {line.split()[2] for line in out.splitlines() if len(line.split()) == 3 and line.split()[1] == "T"}
    assert exported == set(_declared())
