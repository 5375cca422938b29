"""The C ABI: every declared entry point is exported, bound, and validates its arguments.

Runs on the CPU: the library loads without a GPU, and the calls below return
before any HIP runtime call.
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pagedkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for need in ("pa_kv_write", "pa_copy_blocks", "pa_decode_attention", "pa_alloc_create",
                 "pa_seq_append", "pa_seq_fork", "pa_seq_free", "pa_export_tables"):
        assert need in names


def test_every_declared_symbol_is_exported(native):
    out = subprocess.run(["nm", "-D", "--defined-only", native.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (pa_[a-z0-9_]+)$", out, flags=re.M))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"


def test_binding_covers_every_symbol(native):
    assert set(declared_functions()) == set(native.SIGNATURES)
    for name in declared_functions():
        getattr(native.lib(), name)


def test_version_and_error_string(native):
    assert native.pa_version() >= 100
    with pytest.raises(native.PagedKVError) as e:
        native.pa_alloc_create(0, 16)
    assert e.value.code == native.PA_EINVAL
    assert "num_blocks" in native.pa_last_error()


def test_device_entry_points_validate_before_any_hip_call(native):
    L = native.lib()
    # unsupported head_dim / block_size / dtype are rejected on the host
    assert L.pa_kv_write(None, None, None, None, None, 1, 8, 4, 96, 16, 1, None) == native.PA_EUNSUPPORTED
    assert L.pa_kv_write(None, None, None, None, None, 1, 8, 4, 128, 12, 1, None) == native.PA_EUNSUPPORTED
    assert L.pa_kv_write(None, None, None, None, None, 1, 8, 4, 128, 16, 7, None) == native.PA_EINVAL
    assert L.pa_kv_write(None, None, None, None, None, 1, 8, 4, 128, 16, 1, None) == native.PA_EINVAL
    assert L.pa_copy_blocks(None, None, None, 1, 8, 4, 128, 16, 1, None) == native.PA_EINVAL
    assert L.pa_copy_blocks(None, None, None, -1, 8, 4, 128, 16, 1, None) == native.PA_EINVAL
    rc = L.pa_decode_attention(None, None, None, None, None, None, 1, 8, 3, 128, 16, 10, 4, 64, 0,
                               0.1, 1, None, 0, None)
    assert rc == native.PA_EINVAL and "multiple" in native.pa_last_error()
    rc = L.pa_decode_attention(None, None, None, None, None, None, 1, 8, 8, 80, 16, 10, 4, 64, 0,
                               0.1, 1, None, 0, None)
    assert rc == native.PA_EUNSUPPORTED
    rc = L.pa_decode_attention(None, None, None, None, None, None, 1, 8, 8, 128, 16, 10, 4, 64, 24,
                               0.1, 1, None, 0, None)
    assert rc == native.PA_EINVAL
    rc = L.pa_decode_attention(None, None, None, None, None, None, 1, 8, 8, 128, 16, 10, 4, 64, 0,
                               0.1, 1, None, 0, None)
    assert rc == native.PA_EINVAL and "null" in native.pa_last_error()


def test_noalloc_refuses_past_its_workspace_before_any_hip_call(native):
    """The allocation-free decode refuses a launch whose workspace would exceed its built-in
    array (16 MiB), and bad shapes, before touching the device."""
    L = native.lib()
    assert native.pa_decode_noalloc_max_bytes() == 16 << 20
    rc = L.pa_decode_attention_noalloc(None, None, None, None, None, None, 64, 40, 40, 128, 16, 4,
                                       2048, 32768, 16, 0.1, 1, None)
    assert rc == native.PA_EINVAL and "built-in" in native.pa_last_error()
    rc = L.pa_decode_attention_noalloc(None, None, None, None, None, None, 1, 8, 8, 80, 16, 4, 4,
                                       64, 16, 0.1, 1, None)
    assert rc == native.PA_EUNSUPPORTED
    rc = L.pa_decode_attention_noalloc(None, None, None, None, None, None, 1, 8, 8, 128, 16, 4, 4,
                                       64, 16, 0.1, 9, None)
    assert rc == native.PA_EINVAL


def test_shared_block_plan_and_run_validate_before_any_hip_call(native):
    """pa_decode_prefix2_plan and pa_decode_attention_prefix2_run refuse bad counts, shapes,
    widths, a missing workspace and a partial set of new rows on the host."""
    L = native.lib()
    n = None

    def plan(G=2, H=8, Hkv=8, D=128, B=16, members=2, ws=n):
        return L.pa_decode_prefix2_plan(n, n, 4, H, Hkv, D, B, 8, 128, G, n, n, n, 64, 1, n, n, n,
                                        96, members, 1, ws, 0, n)

    def run(kn=n, vn=n, slots=n, G=2, D=128, ws=n):
        return L.pa_decode_attention_prefix2_run(n, n, n, n, kn, vn, slots, n, n, 4, 8, 8, D, 16,
                                                 64, 8, 128, G, 64, 1, 96, 2, 0.1, 1, ws, 0, n)

    assert plan(G=0) == native.PA_EINVAL and ">= 1" in native.pa_last_error()
    assert plan(H=8, Hkv=3) == native.PA_EINVAL and "multiple" in native.pa_last_error()
    assert plan(members=9) == native.PA_EUNSUPPORTED
    assert plan(members=0) == native.PA_EINVAL
    assert plan(D=80) == native.PA_EUNSUPPORTED
    assert plan(B=12) == native.PA_EUNSUPPORTED
    assert plan() == native.PA_EINVAL and "null" in native.pa_last_error()
    assert run(G=0) == native.PA_EINVAL
    assert run(D=96) == native.PA_EUNSUPPORTED
    fake = ctypes.c_void_p(16)
    assert run(kn=fake) == native.PA_EINVAL and "null" in native.pa_last_error()
    assert run(kn=fake, vn=fake) == native.PA_EINVAL and "null" in native.pa_last_error()
    assert run() == native.PA_EINVAL and "null" in native.pa_last_error()
