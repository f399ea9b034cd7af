"""The C-ABI library builds, loads and exports every function that
include/specsam.h declares (no compute calls: this runs without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specsam.h")
LIB = os.path.join(ROOT, "sam_drafting_lossless_amd", "libspecsam.so")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(",
                       src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ["spec_verify", "sam_extend", "sam_draft", "sam_init",
                 "sam_state_bytes", "ss_verify_workspace_bytes",
                 "ss_verify_workspace_bytes_ex", "spec_step",
                 "spec_verify_tree", "ss_tree_workspace_bytes", "sam_draft_tree", "spec_stream", "spec_finish", "sam_extend_draft",
                 "sam_extend_stats", "sam_match",
                 "sam_status", "sam_export",
                 "sam_hash_slots", "ss_version", "ss_last_error_string"]:
        assert want in names


def test_library_exports_every_declared_symbol():
    if not os.path.exists(LIB):
        pytest.fail("libspecsam.so is not built (run __graft_entry__.build())")
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], check=True,
                         capture_output=True, text=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing


def test_library_loads_and_answers_size_queries():
    import torch  # noqa: F401  (share torch's HIP runtime)
    L = ctypes.CDLL(LIB)
    L.ss_verify_workspace_bytes.restype = ctypes.c_size_t
    L.sam_state_bytes.restype = ctypes.c_size_t
    assert L.ss_version() >= 100
    assert L.ss_verify_workspace_bytes(256, 3, 151936) > 256 * 4 * 19 * 16
    assert L.ss_verify_workspace_bytes(256, 17, 151936) == 0  # K > 16
    ex = L.ss_verify_workspace_bytes_ex
    ex.restype = ctypes.c_size_t
    assert ex(256, 3, 151936, 0) == L.ss_verify_workspace_bytes(256, 3, 151936)
    # truncation: per row chunk a 2 KiB histogram and a 1,024-logit segment
    rows = 256 * 4
    assert ex(256, 3, 151936, 1) > ex(256, 3, 151936, 0) + rows * 19 * (2048 + 1024 * 4)
    assert ex(256, 3, 151936, 2) == 0  # unknown flag
    assert L.sam_state_bytes(4, 1000) % 256 == 0
    assert L.sam_state_bytes(0, 1000) == 0
    assert L.sam_hash_slots(9216) == 65536
    # argument errors are reported without touching a device
    rc = L.spec_verify(None, 0, 0, 3, 10, None, None, None, None, None, None,
                       None, None, None, None, None, None, None,
                       ctypes.c_size_t(0), None)
    assert rc == -1
    L.ss_last_error_string.restype = ctypes.c_char_p
    assert b"B >= 1" in L.ss_last_error_string()


def test_binding_constants_match_the_header():
    import sam_drafting_lossless_amd as ssl
    src = open(HEADER).read()
    defs = {k: v.strip() for k, v in
            re.findall(r"#define\s+(SS_\w+)[ \t]+([-() <0-9x]+)", src)}

    def val(name):  # integer literals and shifts only
        assert re.fullmatch(r"[-() <0-9x]+", defs[name])
        return eval(defs[name], {"__builtins__": {}})

    assert val("SS_DTYPE_F32") == ssl.DTYPE_F32
    assert val("SS_DTYPE_BF16") == ssl.DTYPE_BF16
    for n in ("SAM_CAPACITY", "TOKEN_RANGE", "DRAFT_LEN", "NONFINITE",
              "TEMPERATURE", "NO_UNIFORMS"):
        assert val("SS_ST_" + n) == getattr(ssl, "ST_" + n), n
