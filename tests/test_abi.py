"""The C-ABI library builds, loads, and exports every symbol include/ss_sampler.h
declares; host-side argument checks run without a GPU (no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ss_sampler.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ss_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from speculative_decoding_verification_pipeline_amd import sampler
    if not os.path.exists(sampler.LIB_PATH):
        from speculative_decoding_verification_pipeline_amd import build
        build.build()
    return sampler.load_library()


def test_header_declares_the_entry_points():
    fns = declared_functions()
    for f in ("ss_sampler_create", "ss_sample", "ss_spec_verify", "ss_spec_verify_scatter",
              "ss_tree_verify", "ss_lmhead_sample", "ss_lmhead_sample_params",
              "ss_sample_noalloc"):
        assert f in fns


def test_library_exports_every_declared_symbol(lib):
    from speculative_decoding_verification_pipeline_amd import sampler
    out = subprocess.run(["nm", "-D", "--defined-only", sampler.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for f in declared_functions():
        assert f in exported, f
        assert hasattr(lib, f)
    assert set(sampler.EXPORTED) <= set(declared_functions())


def test_status_strings(lib):
    for st in (0, -1, -2, -3, -4):
        assert lib.ss_status_string(st)
    assert lib.ss_status_string(0) == b"ok"


def test_create_rejects_bad_limits_before_touching_hip(lib):
    from speculative_decoding_verification_pipeline_amd import sampler
    h = ctypes.c_void_p()
    bad = [sampler.Config(0, 100, 0, 0, 0), sampler.Config(4, 0, 0, 0, 0),
           sampler.Config(4, 300000, 0, 0, 0), sampler.Config(4, 100, 64, 0, 0),
           sampler.Config(4, 100, 0, 100, 0), sampler.Config(4, 100, 0, 0, -1)]
    for cfg in bad:
        assert lib.ss_sampler_create(ctypes.byref(cfg), ctypes.byref(h)) == sampler.SS_ERR_INVALID_ARG
    assert lib.ss_sampler_create(None, ctypes.byref(h)) == sampler.SS_ERR_INVALID_ARG


def test_calls_reject_null_handle(lib):
    from speculative_decoding_verification_pipeline_amd import sampler
    p = sampler.CParams()
    assert lib.ss_sample(None, None, 0, 0, 1, ctypes.byref(p), None, None, None) == \
        sampler.SS_ERR_INVALID_ARG
    assert lib.ss_spec_verify(None, None, 0, 0, None, 0, None, 1, 1, ctypes.byref(p), None,
                              None, None) == sampler.SS_ERR_INVALID_ARG
    assert lib.ss_lmhead_sample(None, None, None, 1, None, None, None, 0, None, None,
                                None) == sampler.SS_ERR_INVALID_ARG
    assert lib.ss_tree_verify(None, None, 0, 0, None, None, 1, 2, ctypes.byref(p), None, None,
                              None, None) == sampler.SS_ERR_INVALID_ARG
    assert lib.ss_spec_verify_scatter(None, None, 0, 0, None, 0, None, 1, 1, ctypes.byref(p), None,
                                      None, None, None) == sampler.SS_ERR_INVALID_ARG
    assert lib.ss_lmhead_sample_params(None, None, None, 1, ctypes.byref(p), None, None,
                                       None) == sampler.SS_ERR_INVALID_ARG
    assert lib.ss_sampler_workspace_bytes(None) == 0
    assert lib.ss_sampler_set_launch_events(None, None, 0) == sampler.SS_ERR_INVALID_ARG
    lib.ss_sampler_destroy(None)
