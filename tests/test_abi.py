"""The C ABI library loads on a machine without a GPU and exports every entry
point include/pe.h declares.  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pe.h")
LIB = os.path.join(ROOT, "drafting_pe_prepare_amd", "libpe.so")


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_step_calls():
    names = declared()
    for n in ("pe_prepare", "pe_gather_hidden", "pe_draft_forward", "pe_verify",
              "pe_step_graph", "pe_create", "pe_destroy", "pe_get_device_error"):
        assert n in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libpe.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    for n in declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pe_[a-z_]+)$", out, flags=re.M))
    assert set(declared()) <= exported


@pytest.mark.skipif(not os.path.exists(LIB), reason="libpe.so not built")
def test_library_is_gfx950_only():
    """The embedded offload bundle names only gfx950 code objects."""
    blob = open(LIB, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa--(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}, targets


def test_binding_names_match_the_abi():
    from drafting_pe_prepare_amd import binding
    for n in ("pe_prepare", "pe_gather_hidden", "pe_draft_forward", "pe_verify",
              "pe_step_graph", "pe_get_device_error"):
        assert callable(getattr(binding, n))
    assert set(binding.EXPORTS) <= set(declared())


@pytest.mark.skipif(not os.path.exists(LIB), reason="libpe.so not built")
def test_binding_declares_argument_types_of_every_entry_point():
    """Without argtypes ctypes passes a Python int as a 32-bit C int and
    silently truncates 64-bit device pointers, so every entry point must carry
    argument types, as many as its prototype in the header has parameters."""
    from drafting_pe_prepare_amd import binding
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = dict(re.findall(r"\b(pe_[a-z_]+)\s*\(([^)]*)\)\s*;", text))
    assert set(binding.EXPORTS) == set(declared()) == set(protos)
    lib = binding.load()
    for name, params in protos.items():
        n = 0 if params.strip() in ("", "void") else params.count(",") + 1
        at = getattr(lib, name).argtypes
        assert at is not None, f"{name} has no argtypes"
        assert len(at) == n, (name, len(at), n)
