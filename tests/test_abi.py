"""The C-ABI library loads, exports every function include/*.h declares, and
its host-side argument checks reject bad calls before any HIP work. Runs
without a GPU: every call here returns before the library touches a device."""
import ctypes
import glob
import os
import re

import pytest

import temperature_softmax_vocabulary_amd as tsv
from temperature_softmax_vocabulary_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_A = 0x10000000       # never dereferenced: checks fail before any device access
FAKE_B = 0x20000000
INVALID = binding.TS_ERR_INVALID_ARGUMENT


def _declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(ts_\w+)\s*\(", text, flags=re.M))
    return names


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail(f"{binding.LIB_PATH} missing: build it with python -m temperature_softmax_vocabulary_amd.build")
    return binding.lib()


def test_every_declared_symbol_is_exported(L):
    declared = _declared_functions()
    assert {"ts_softmax", "ts_sample", "ts_reserve", "ts_status_string"} <= declared
    for name in sorted(declared):
        assert hasattr(L, name), f"{name} declared in include/ but not exported"
    # and the binding wraps exactly the declared set
    assert set(binding.SIGNATURES) == declared


def test_abi_version_and_status_strings(L):
    assert tsv.ts_abi_version() == 1
    for s in range(6):
        assert tsv.ts_status_string(s).startswith("TS_")
    assert "unknown" in tsv.ts_status_string(99)


@pytest.mark.parametrize("B,V", [(-1, 10), (1, 0), (1, -5), (1, 2**31), (2**40, 2**31 - 1)])
def test_softmax_rejects_bad_sizes(L, B, V):
    assert L.ts_softmax(FAKE_A, FAKE_B, B, V, FAKE_A + (1 << 40), None) == INVALID


def test_softmax_zero_rows_is_a_noop(L):
    assert L.ts_softmax(None, None, 0, 151936, None, None) == binding.TS_OK


def test_softmax_rejects_null_pointers(L):
    assert L.ts_softmax(None, FAKE_B, 3, 100, FAKE_A, None) == INVALID
    assert L.ts_softmax(FAKE_A, None, 3, 100, FAKE_A, None) == INVALID
    assert L.ts_softmax(FAKE_A, FAKE_B, 3, 100, None, None) == INVALID


def test_softmax_rejects_partial_overlap_but_not_exact_alias_check(L):
    # out shifted by one float inside logits: rejected
    assert L.ts_softmax(FAKE_A, FAKE_B, 2, 100, FAKE_A + 4, None) == INVALID
    # out overlapping temps: rejected
    assert L.ts_softmax(FAKE_A, FAKE_B + 8, 2, 100, FAKE_B, None) == INVALID


def test_softmax_variant_rejects_bad_variant_or_chunk(L):
    assert L.ts_softmax_variant(FAKE_A, FAKE_B, None, 2, 100, FAKE_A, 7, 0, None) == INVALID
    assert L.ts_softmax_variant(FAKE_A, FAKE_B, None, 2, 100, FAKE_A, 1, 3000, None) == INVALID
    assert L.ts_softmax_variant(FAKE_A, FAKE_B, None, 2, 100, FAKE_A, 1, 32768, None) == INVALID


def test_masked_argument_checks(L):
    # the mask is required, and may not overlap the output
    assert L.ts_softmax_masked(FAKE_A, FAKE_B, None, 2, 100, FAKE_A + (1 << 30), None) == INVALID
    assert L.ts_softmax_masked(FAKE_A, FAKE_B, FAKE_A + (1 << 30) + 64, 2, 100, FAKE_A + (1 << 30), None) == INVALID
    assert L.ts_softmax_masked(None, None, None, 0, 100, None, None) == binding.TS_OK
    assert L.ts_softmax_sample(FAKE_A, FAKE_B, FAKE_A + (1 << 31), FAKE_B + 64, 2, 100, 4, None,
                               FAKE_A + (1 << 31) + 4, None) == INVALID


def test_sample_argument_checks(L):
    assert L.ts_sample(FAKE_A, FAKE_B, 1, 10, -1, FAKE_A + (1 << 30), None) == INVALID
    assert L.ts_sample(None, FAKE_B, 1, 10, 4, FAKE_A, None) == INVALID
    assert L.ts_sample(FAKE_A, FAKE_B, 0, 10, 4, None, None) == binding.TS_OK
    assert L.ts_sample(FAKE_A, FAKE_B, 2, 10, 0, None, None) == binding.TS_OK
    # ids written over the probs: rejected
    assert L.ts_sample(FAKE_A, FAKE_B, 2, 10, 4, FAKE_A + 16, None) == INVALID
    assert L.ts_sample(FAKE_A, FAKE_B, 2, 10, 4, FAKE_B + 4, None) == INVALID


def test_reserve_plan_copy_argument_checks(L):
    assert L.ts_reserve(-1, 10, None) == INVALID
    assert L.ts_reserve(1, 0, None) == INVALID
    v = ctypes.c_int32()
    assert L.ts_plan(1, 10, None, ctypes.byref(v)) == INVALID
    assert L.ts_plan(-1, 10, ctypes.byref(v), ctypes.byref(v)) == INVALID
    assert L.ts_copy_f32(FAKE_A, FAKE_A + 8, 100, None) == INVALID
    assert L.ts_copy_f32(FAKE_A, FAKE_B, -1, None) == INVALID
    assert L.ts_copy_f32(None, None, 0, None) == binding.TS_OK
    assert L.ts_device_errors(None, None) == INVALID
    assert L.ts_debug_set_spin_limit(0) == binding.TS_OK


def test_binding_raises_value_error_on_invalid_argument():
    with pytest.raises(ValueError):
        binding._check(INVALID)
    with pytest.raises(binding.TsError):
        binding._check(binding.TS_ERR_HIP)


def test_host_tensors_are_refused_without_a_library_call():
    # the binding checks devices before it calls into the library: host tensors
    # never reach a kernel (and there is no host path to fall back to)
    import torch
    import temperature_softmax_vocabulary_amd as tsv
    x, t, u = torch.randn(2, 10), torch.ones(2), torch.rand(2, 3)
    for call in (lambda: tsv.ts_softmax(x, t), lambda: tsv.ts_sample(x, u),
                 lambda: tsv.ts_softmax_sample(x, t, u), lambda: tsv.ts_softmax_masked(x, t, None)):
        with pytest.raises(ValueError, match="HIP device"):
            call()


def test_product_path_has_no_oracle_or_cpu_fallback():
    # The package never imports the oracle, and nothing under it names a CPU
    # softmax route: the binding only marshals arguments into the library.
    pkg = os.path.join(ROOT, "temperature_softmax_vocabulary_amd")
    for path in glob.glob(os.path.join(pkg, "**", "*.py"), recursive=True):
        text = open(path).read()
        assert "oracle" not in text.replace("oracle's", ""), path
        assert "torch.softmax" not in text and "np.exp" not in text, path


@pytest.mark.parametrize("B,V,expect", [
    (1, 16384, (binding.TS_VARIANT_ROWWISE, 0)),            # the row fits one workgroup's registers
    (64, 5003, (binding.TS_VARIANT_ROWWISE, 0)),
    (767, 16384, (binding.TS_VARIANT_ROWWISE, 0)),           # short rows: one workgroup per row ...
    (768, 16384, (binding.TS_VARIANT_FUSED, 8192)),          # ... except 768..2048 rows of 4096..16384
    (2048, 4096, (binding.TS_VARIANT_FUSED, 4096)),
    (2049, 4096, (binding.TS_VARIANT_ROWWISE, 0)),
    (1024, 4095, (binding.TS_VARIANT_ROWWISE, 0)),
    (127, 20480, (binding.TS_VARIANT_FUSED, 8192)),          # 16385..32768 columns: fused, but one
    (128, 20480, (binding.TS_VARIANT_ROWWISE, 0)),           # workgroup per row from 128 rows up
    (128, 20484, (binding.TS_VARIANT_FUSED, 8192)),          # to 20480 columns ...
    (2047, 32768, (binding.TS_VARIANT_FUSED, 8192)),
    (2048, 32768, (binding.TS_VARIANT_ROWWISE, 0)),          # ... and from 2048 rows up to 32768
    (2048, 32772, (binding.TS_VARIANT_FUSED, 8192)),
    (1, 151936, (binding.TS_VARIANT_FUSED, 4096)),           # B*V <= 2^20: latency-bound, small chunks
    (4, 262144, (binding.TS_VARIANT_FUSED, 4096)),           # exactly 2^20
    (8, 201088, (binding.TS_VARIANT_FUSED, 8192)),           # 1.6e6 elements
    (64, 32768, (binding.TS_VARIANT_FUSED, 4096)),           # short rows: 4096 up to 2^21
    (65, 32768, (binding.TS_VARIANT_FUSED, 8192)),
    (16, 201088, (binding.TS_VARIANT_FUSED, 8192)),
    (64, 262144, (binding.TS_VARIANT_FUSED, 8192)),          # the bench workload
    (2, 2 * 1024 * 1024 + 4099, (binding.TS_VARIANT_FUSED, 16384)),   # > 256 chunks of 8192
    (2, 4 * 1024 * 1024 + 1000, (binding.TS_VARIANT_SPLIT, 16384)),   # > 256 chunks of 16384
])
def test_work_split_table(L, B, V, expect):
    # the measured table of the work split (host only, no device needed)
    v, c = ctypes.c_int32(), ctypes.c_int32()
    assert L.ts_plan(B, V, ctypes.byref(v), ctypes.byref(c)) == binding.TS_OK
    assert (v.value, c.value) == expect


C_PROGRAM = r"""
#include "tsoftmax.h"
#include "tsoftmax_measure.h"
#include <stdio.h>

/* every entry point, taken by address with its declared C type */
int main(void) {
    ts_status (*softmax)(const float*, const float*, int64_t, int64_t, float*, hipStream_t) = ts_softmax;
    ts_status (*masked)(const float*, const float*, const uint32_t*, int64_t, int64_t, float*, hipStream_t) =
        ts_softmax_masked;
    ts_status (*variant)(const float*, const float*, const uint32_t*, int64_t, int64_t, float*, int32_t, int32_t,
                         hipStream_t) = ts_softmax_variant;
    ts_status (*plan)(int64_t, int64_t, int32_t*, int32_t*) = ts_plan;
    ts_status (*sample)(const float*, const float*, int64_t, int64_t, int64_t, int32_t*, hipStream_t) = ts_sample;
    ts_status (*fused)(const float*, const float*, const uint32_t*, const float*, int64_t, int64_t, int64_t, float*,
                       int32_t*, hipStream_t) = ts_softmax_sample;
    ts_status (*reserve)(int64_t, int64_t, hipStream_t) = ts_reserve;
    ts_status (*errors)(hipStream_t, uint32_t*) = ts_device_errors;
    const char* (*text)(ts_status) = ts_status_string;
    int32_t (*version)(void) = ts_abi_version;
    ts_status (*copy)(const float*, float*, int64_t, hipStream_t) = ts_copy_f32;
    ts_status (*spin)(uint32_t) = ts_debug_set_spin_limit;
    ts_status (*cap)(int64_t) = ts_debug_set_resident_cap;
    ts_status (*mem)(int32_t, int32_t*, int32_t*) = ts_device_memory_params;
    void* all[] = {(void*)softmax, (void*)masked, (void*)variant, (void*)plan, (void*)sample, (void*)fused,
                   (void*)reserve, (void*)errors, (void*)text, (void*)version, (void*)copy, (void*)spin,
                   (void*)cap, (void*)mem};
    printf("%d %d\n", (int)(sizeof all / sizeof all[0]), TSOFTMAX_ABI_VERSION);
    return 0;
}
"""


def test_headers_are_c_and_link_against_the_library(tmp_path):
    # The boundary is a C ABI: the public headers compile as C11 (no C++), and a
    # C program that takes every entry point links against libtsoftmax.so. It is
    # compiled and linked only: nothing runs on a GPU here.
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    if not os.path.exists(binding.LIB_PATH):
        pytest.fail(f"{binding.LIB_PATH} missing")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [cc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           f"-I{os.path.join(ROOT, 'include')}", f"-I{os.path.join(rocm, 'include')}",
           str(src), "-o", str(tmp_path / "abi"), binding.LIB_PATH, f"-Wl,-rpath,{os.path.dirname(binding.LIB_PATH)}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
