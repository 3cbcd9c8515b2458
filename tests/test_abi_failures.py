"""Host-side robustness of the C ABI, on the CPU.

* A launch the HIP runtime refuses reaches the caller as DQKV_ERR_HIP: every
  entry point that launches kernels is called with valid sizes in a child
  process whose HIP runtime sees no device (HIP_VISIBLE_DEVICES=-1), so the
  launch itself fails; the child first checks that it sees no device and
  otherwise launches nothing.
* Seeded fuzzing of every entry point's argument checks in such a child:
  random sizes (negative, zero, odd, huge), scales (negative, NaN, inf),
  null, aligned and misaligned device pointers and workspace sizes; every
  call returns one of the documented status codes, and the child ends
  normally.
* The ABI's host code (argument checks, planning, workspace layout) runs its
  tests under AddressSanitizer and UndefinedBehaviorSanitizer: a build of
  api.hip with host-side sanitizers, loaded into a child process that
  preloads the ASan runtime.
"""

import os
import subprocess
import sys
import textwrap

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
dq = pytest.importorskip("asymmetric_head_kv_amd")

NO_DEVICE = {"HIP_VISIBLE_DEVICES": "-1", "ROCR_VISIBLE_DEVICES": "-1",
             "CUDA_VISIBLE_DEVICES": "-1"}

CHILD = textwrap.dedent('''
    import ctypes, sys
    sys.path.insert(0, ROOT)
    hip = ctypes.CDLL("libamdhip64.so")
    n = ctypes.c_int(-1)
    hip.hipGetDeviceCount(ctypes.byref(n))
    if n.value > 0:
        print("SKIP: a device is visible"); sys.exit(0)
    import asymmetric_head_kv_amd as dq
    lib = dq.load()
    F = 1 << 20          # aligned, never dereferenced: every launch is refused
    ws = dq.decode_workspace_bytes(16, 4, 16, 64, 128, 1, 1024)
    sws = dq.selective_workspace_bytes(16, 4, 16, 64, 128, 1, 1024, 100)
    calls = {
        "kv_append": lambda: lib.kv_append(16, 4, 16, 64, 128, 1, 1, 1, 1024, F, F, F, F, F, None),
        "diffqkv_decode": lambda: lib.diffqkv_decode(16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0,
                                                     F, F, F, F, F, None, 0, F, ws, None),
        "diffqkv_decode_append": lambda: lib.diffqkv_decode_append(
            16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, F, F, F, F, F, F, None, 0, F, ws, None),
        "diffqkv_decode_append_noalloc": lambda: lib.diffqkv_decode_append_noalloc(
            16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, F, F, F, F, F, F, None, 0, None),
        "diffqkv_decode_split": lambda: lib.diffqkv_decode_split(
            16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, None, None, F, F, F, 0, F, ws, None),
        "diffqkv_decode_combine": lambda: lib.diffqkv_decode_combine(
            16, 4, 16, 64, 128, 1, 1, 1024, 1024, F, F, None, 0, F, ws, None),
        "diffqkv_prefill": lambda: lib.diffqkv_prefill(16, 4, 16, 64, 128, 1, 1, 64, 1024, 0.0,
                                                       F, F, F, F, F, None, None, 0, None),
        "diffqkv_prefill_paged": lambda: lib.diffqkv_prefill_paged(
            16, 4, 16, 64, 128, 1, 1, 64, 64, 16, 16, 0.0, F, F, F, F, F, F, None, None, 0, None),
        "diffqkv_decode_selective": lambda: lib.diffqkv_decode_selective(
            16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, 100, F, None, None, F, F, F, F, None,
            None, F, sws, None),
        "diffqkv_decode_selective_paged": lambda: lib.diffqkv_decode_selective_paged(
            16, 4, 16, 64, 128, 1, 1, 64, 16, 16, 1024, 0.0, 100, F, None, None, F, F, F, F, F,
            None, None, F, sws, None),
        "kv_append_paged": lambda: lib.kv_append_paged(16, 4, 16, 64, 128, 1, 1, 1, 64, 16, 16,
                                                       F, F, F, F, F, F, None),
        "diffqkv_decode_paged": lambda: lib.diffqkv_decode_paged(
            16, 4, 16, 64, 128, 1, 1, 64, 16, 16, 1024, 0.0, F, None, None, F, F, F, F, F, None,
            0, F, ws, None),
        "kv_group_sharing": lambda: lib.kv_group_sharing(16, 4, 16, 64, 128, 1, 1, 1024, F, F, F,
                                                         F, None),
        "augq_pack": lambda: lib.augq_pack(64, 64, F, F, None),
        "augq_forward": lambda: lib.augq_forward(1, 1024, 1024, 256, F, F, F, F, F, F, 1 << 20,
                                                 None),
    }
    bad = {}
    for name, fn in calls.items():
        st = fn()
        if st != -5:
            bad[name] = st
    # The failure is reported, not remembered: a later call's own checks
    # still decide its status.
    after = lib.diffqkv_decode(16, 3, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, F, F, F, F, None,
                               0, F, ws, None)
    print("RESULT", len(calls), bad, after, lib.dqkv_status_str(-5).decode())
''')


def _child(extra_env=None):
    env = dict(os.environ, **NO_DEVICE, **(extra_env or {}))
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + CHILD], env=env,
                       capture_output=True, text=True, timeout=300)
    return r


def test_refused_launch_reaches_the_caller_as_err_hip():
    if not os.path.exists(dq.lib_path):
        pytest.skip("libdiffqkv.so not built")
    r = _child()
    assert r.returncode == 0, r.stderr[-3000:]
    out = r.stdout.strip().splitlines()
    if out and out[-1].startswith("SKIP"):
        pytest.skip(out[-1])
    last = out[-1]
    assert last.startswith("RESULT 15 {} -2 DQKV_ERR_HIP"), last


def test_abi_host_code_under_asan_and_ubsan():
    if not os.path.exists("/opt/rocm/llvm/bin/clang++"):
        pytest.skip("no ROCm clang++ for the sanitizer build")
    from asymmetric_head_kv_amd.build_sanitized import asan_runtime, build_sanitized
    lib = build_sanitized()
    env = dict(os.environ, **NO_DEVICE, DQKV_LIBRARY=lib, LD_PRELOAD=asan_runtime(),
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    # The library under test carries the sanitizer instrumentation.
    nm = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in nm and "__ubsan_handle" in nm
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py"),
                        os.path.join(ROOT, "tests", "test_abi_failures.py"),
                        "-k", "not asan"],
                       env=env, capture_output=True, text=True, timeout=600, cwd=ROOT)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "ERROR: AddressSanitizer" not in r.stderr and "runtime error:" not in r.stderr


FUZZ = textwrap.dedent('''
    import ctypes, sys, collections
    import numpy as np
    sys.path.insert(0, ROOT)
    hip = ctypes.CDLL("libamdhip64.so")
    n = ctypes.c_int(-1)
    hip.hipGetDeviceCount(ctypes.byref(n))
    if n.value > 0:
        print("SKIP: a device is visible"); sys.exit(0)
    import asymmetric_head_kv_amd as dq
    lib = dq.load()
    rng = np.random.default_rng(20261204)
    F = 1 << 20                      # aligned, never dereferenced
    INTS = [0, 1, 2, 3, 4, 7, 16, 32, 63, 64, 65, 100, 128, 256, 1000, 1024, 4096, 65535,
            65536, 1 << 20, 2**31 - 1, -1, -2, -64, -(2**31)]
    SCALES = [0.0, 0.125, 1.0, -1.0, -0.0, float("nan"), float("inf"), float("-inf"), 1e-30]
    SIZES = [0, 1, 16, 255, 4096, 1 << 20, 1 << 30, 1 << 40, 2**64 - 1]
    codes = collections.Counter()
    calls = 0
    for name, (res, args) in dq.SIGNATURES.items():
        fn = getattr(lib, name)
        for _ in range(200):
            vals = []
            for k, a in enumerate(args):
                last = k == len(args) - 1
                if a is ctypes.c_int32:
                    vals.append(int(INTS[rng.integers(len(INTS))]) if rng.random() < 0.8
                                else int(rng.integers(-5, 300)))
                elif a is ctypes.c_float:
                    vals.append(SCALES[rng.integers(len(SCALES))])
                elif a is ctypes.c_size_t:
                    vals.append(SIZES[rng.integers(len(SIZES))])
                elif a is ctypes.c_void_p:
                    # the last pointer of a launching entry point is its stream: the default
                    vals.append(None if last else [None, F, F + 2, F][rng.integers(4)])
                else:                    # a host out-parameter
                    vals.append(None if rng.random() < 0.2 else ctypes.byref(a._type_()))
            if name == "dqkv_status_str":
                r = fn(*vals)
                assert r is not None
                continue
            st = fn(*vals)
            calls += 1
            codes[st] += 1
            assert st in (0, -1, -2, -3, -4, -5, -6), (name, vals, st)
    # Valid calls with one or two arguments replaced: each check is reached
    # on its own, past the ones before it.
    ws = dq.decode_workspace_bytes(16, 4, 16, 64, 128, 1, 1024)
    sws = dq.selective_workspace_bytes(16, 4, 16, 64, 128, 1, 1024, 100)
    base = {
        "kv_append": (16, 4, 16, 64, 128, 1, 1, 1, 1024, F, F, F, F, F, None),
        "diffqkv_decode": (16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, F, F, F, F, None, 0, F,
                           ws, None),
        "diffqkv_decode_append": (16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, F, F, F, F, F, F,
                                  None, 0, F, ws, None),
        "diffqkv_decode_append_noalloc": (16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, F, F, F,
                                          F, F, F, None, 0, None),
        "diffqkv_decode_split": (16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, F, None, None, F, F,
                                 F, 0, F, ws, None),
        "diffqkv_decode_combine": (16, 4, 16, 64, 128, 1, 1, 1024, 1024, F, F, None, 0, F, ws,
                                   None),
        "diffqkv_prefill": (16, 4, 16, 64, 128, 1, 1, 64, 1024, 0.0, F, F, F, F, F, None, None,
                            0, None),
        "diffqkv_prefill_paged": (16, 4, 16, 64, 128, 1, 1, 64, 64, 16, 16, 0.0, F, F, F, F, F,
                                  F, None, None, 0, None),
        "diffqkv_decode_selective": (16, 4, 16, 64, 128, 1, 1, 1024, 1024, 0.0, 100, F, None,
                                     None, F, F, F, F, None, None, F, sws, None),
        "diffqkv_decode_selective_paged": (16, 4, 16, 64, 128, 1, 1, 64, 16, 16, 1024, 0.0, 100,
                                           F, None, None, F, F, F, F, F, None, None, F, sws,
                                           None),
        "kv_append_paged": (16, 4, 16, 64, 128, 1, 1, 1, 64, 16, 16, F, F, F, F, F, F, None),
        "diffqkv_decode_paged": (16, 4, 16, 64, 128, 1, 1, 64, 16, 16, 1024, 0.0, F, None, None,
                                 F, F, F, F, F, None, 0, F, ws, None),
        "kv_group_sharing": (16, 4, 16, 64, 128, 1, 1, 1024, F, F, F, F, None),
        "augq_pack": (64, 64, F, F, None),
        "augq_forward": (1, 1024, 1024, 256, F, F, F, F, F, F, 1 << 20, None),
    }
    mutated = 0
    for name, vals0 in base.items():
        fn = getattr(lib, name)
        args = dq.SIGNATURES[name][1]
        assert len(args) == len(vals0), name
        for _ in range(150):
            vals = list(vals0)
            for k in rng.choice(len(vals) - 1, size=int(rng.integers(1, 3)), replace=False):
                a = args[k]
                if a is ctypes.c_int32:
                    vals[k] = int(INTS[rng.integers(len(INTS))])
                elif a is ctypes.c_float:
                    vals[k] = SCALES[rng.integers(len(SCALES))]
                elif a is ctypes.c_size_t:
                    vals[k] = SIZES[rng.integers(len(SIZES))]
                else:
                    vals[k] = [None, F, F + 2][rng.integers(3)]
            st = fn(*vals)
            mutated += 1
            codes[st] += 1
            assert st in (0, -1, -2, -3, -4, -5, -6), (name, vals, st)
    print("RESULT", calls + mutated, dict(sorted(codes.items())))
''')


def test_fuzzed_arguments_give_documented_status_codes():
    if not os.path.exists(dq.lib_path):
        pytest.skip("libdiffqkv.so not built")
    env = dict(os.environ, **NO_DEVICE)
    r = subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + FUZZ], env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    out = r.stdout.strip().splitlines()
    if out and out[-1].startswith("SKIP"):
        pytest.skip(out[-1])
    assert out[-1].startswith("RESULT"), out[-5:]
    calls, codes = out[-1].split(" ", 2)[1:]
    assert int(calls) == 200 * (len(dq.SIGNATURES) - 1) + 150 * 15
