"""Host-side checks that need no GPU: the C-ABI library loads and exports every
symbol include/lora.h declares, argument validation that fails before any
device call, the public struct layout, and the slot book / tenant ledger
(compiled on its own with g++)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lora.h")


def _lora():
    from rank_adapter_gemm_token_amd import lora
    return lora


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared_functions() == sorted(_lora().EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lora().raw_lib()
    out = subprocess.run(["nm", "-D", "--defined-only", _lora().LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (lora_\w+)", out))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_has_gfx950_code():
    out = subprocess.run(["/opt/rocm/llvm/bin/llvm-readelf", "-S", _lora().LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    assert ".hip_fatbin" in out
    blob = open(_lora().LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob


def test_strerror_texts():
    L = _lora()
    codes = [L.LORA_OK, L.LORA_EINVAL, L.LORA_ETOKENS, L.LORA_ESLOT_BUSY, L.LORA_ESLOT_EMPTY,
             L.LORA_ERANK, L.LORA_EALPHA, L.LORA_EQUOTA, L.LORA_EMISMATCH, L.LORA_ENOMEM, L.LORA_EHIP]
    texts = [L.lora_strerror(c) for c in codes]
    assert len(set(texts)) == len(texts)
    assert L.lora_strerror(-999) == "unknown status"


def test_validation_before_device_use():
    lib = _lora().raw_lib()
    L = _lora()
    h = ctypes.c_void_p()
    # Bad sizes / dtype / null output: refused before touching the device.
    assert lib.lora_pool_create(0, 64, 8, 4, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(64, 64, 0, 4, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(64, 64, 65, 4, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(64, 64, 8, 0, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(64, 64, 8, 1025, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(64, 64, 8, 4, 0, 1, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(64, 64, 8, 4, 16, 7, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_pool_create(96, 64, 8, 4, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL  # fp16 needs %64
    assert lib.lora_pool_create(64, 64, 8, 4, 16, 1, None) == L.LORA_EINVAL
    # x, W or y of 4 GiB or more: the kernels' 32-bit byte offsets could not reach them.
    assert lib.lora_pool_create(65536, 32768, 8, 4, 16, 1, ctypes.byref(h)) == L.LORA_EINVAL  # W 4 GiB
    assert lib.lora_pool_create(4096, 64, 8, 4, 524288, 1, ctypes.byref(h)) == L.LORA_EINVAL  # x 4 GiB
    assert lib.lora_pool_create(64, 4096, 8, 4, 524288, 1, ctypes.byref(h)) == L.LORA_EINVAL  # y 4 GiB
    assert lib.lora_pool_create(32768, 32768, 8, 4, 16, 0, ctypes.byref(h)) == L.LORA_EINVAL  # fp32 W 4 GiB
    assert lib.lora_last_routing(None, None, None, None, None, None) == L.LORA_EINVAL
    # Null pool handles.
    assert lib.lora_pool_destroy(None) == L.LORA_OK
    assert lib.lora_apply(None, None, None, None, 4, None, None) == L.LORA_EINVAL
    assert lib.lora_register(None, 0, 0, None, None, 8, ctypes.c_float(16.0), None) == L.LORA_EINVAL
    assert lib.lora_unregister(None, 0) == L.LORA_EINVAL
    assert lib.lora_set_tenant_quota(None, 0, 10) == L.LORA_EINVAL
    assert lib.lora_set_policy(None, 0, 16) == L.LORA_EINVAL
    assert lib.lora_set_shrink_wait_polls(None, 0) == L.LORA_EINVAL
    assert lib.lora_route(None, None, 0, None, None, None, None, None, None) == L.LORA_EINVAL
    s = L.lora_stats()
    assert lib.lora_pool_stats(None, ctypes.byref(s)) == L.LORA_EINVAL
    v = ctypes.c_uint64()
    assert lib.lora_poll_errors(None, ctypes.byref(v)) == L.LORA_EINVAL
    assert lib.lora_tenant_bytes(None, 0, ctypes.byref(v)) == L.LORA_EINVAL
    # Plans: bad sizes and null handles are refused before the device.
    assert lib.lora_plan_create(0, 4, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_plan_create(16, 0, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_plan_create(16, 1025, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_plan_create(16, 4, None) == L.LORA_EINVAL
    assert lib.lora_plan_destroy(None) == L.LORA_OK
    assert lib.lora_plan_route(None, None, None, 4, None) == L.LORA_EINVAL
    assert lib.lora_apply_routed(None, None, None, None, None, None) == L.LORA_EINVAL
    # Loader: zero capacity, null handles.
    assert lib.lora_loader_create(0, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_loader_create(1024, None) == L.LORA_EINVAL
    assert lib.lora_loader_destroy(None) == L.LORA_OK
    t = ctypes.c_uint64()
    assert lib.lora_load_async(None, None, 0, 0, None, None, 8, ctypes.c_float(16.0), ctypes.byref(t)) == L.LORA_EINVAL
    d = ctypes.c_int()
    assert lib.lora_load_poll(None, 1, ctypes.byref(d)) == L.LORA_EINVAL
    assert lib.lora_load_wait(None, 1) == L.LORA_EINVAL
    # Residency: null handles.
    assert lib.lora_residency_create(None, None, 2, ctypes.byref(h)) == L.LORA_EINVAL
    assert lib.lora_residency_destroy(None) == L.LORA_OK
    assert lib.lora_residency_set_share(None, 0, 1) == L.LORA_EINVAL
    sl = ctypes.c_int()
    assert lib.lora_residency_acquire(None, 1, 0, None, None, 8, ctypes.c_float(16.0), ctypes.byref(sl),
                                      ctypes.byref(t)) == L.LORA_EINVAL
    assert lib.lora_residency_release(None, 1) == L.LORA_EINVAL


def test_stats_struct_layout_matches_header(tmp_path):
    L = _lora()
    fields = [n for n, _ in L.lora_stats._fields_]
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "lora.h"', 'int main(void){',
             'printf("%zu\\n", sizeof(lora_stats));']
    lines += ['printf("%%zu\\n", offsetof(lora_stats, %s));' % f for f in fields]
    lines += ['return 0;}']
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)], check=True)
    got = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(L.lora_stats)
    assert got[1:] == [getattr(L.lora_stats, f).offset for f in fields]


# The pure C++ parts of the host runtime (slot book and tenant ledger, LRU-K
# residency policy), built plain and under AddressSanitizer + UBSan (host code
# only; any report aborts the run).
SANITIZE = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]


def _native_check(tmp_path, name, src, flags):
    exe = tmp_path / name
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", *flags, "-o", str(exe),
                    os.path.join(ROOT, "tests", "native", name + ".cpp"),
                    os.path.join(ROOT, "rank_adapter_gemm_token_amd", "csrc", src)],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr


@pytest.mark.parametrize("flags", [[], SANITIZE], ids=["plain", "asan_ubsan"])
def test_slot_book_and_ledger(tmp_path, flags):
    _native_check(tmp_path, "ledger_check", "ledger.cpp", flags)


@pytest.mark.parametrize("flags", [[], SANITIZE], ids=["plain", "asan_ubsan"])
def test_residency_policy(tmp_path, flags):
    _native_check(tmp_path, "residency_check", "residency.cpp", flags)
