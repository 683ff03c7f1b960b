"""Sanitizer runs of the host code, on the CPU (no GPU, no kernel launched).

* The host library (config checks, workspace layout, queue planner, the
  C-ABI entry points' validation) built with AddressSanitizer and
  UndefinedBehaviorSanitizer on its host side only (the device code is built
  as usual, and nothing here launches a kernel), with the ABI tests of
  test_abi_host.py run against it in a child process.
* A fuzz driver (tests/sanitize/plan_fuzz.cpp) that runs the queue planner
  over thousands of random configs and batches under the same sanitizers,
  with every output array sized exactly, checking the queue's invariants;
  its queues are also compared with the oracle's.
* A CPU model of the resident loop's step protocol
  (tests/sanitize/loop_protocol.cpp) under ThreadSanitizer: host and
  workgroup threads exchange epochs, slot counters and outputs as the
  resident kernel does; every unit of every step must be done exactly once
  and no plain memory may be touched without a happens-before edge.  The same
  model with the slot re-armed too early (a mistake an earlier version of the
  kernel made) must be caught.
"""

import os
import subprocess
import sys

import numpy as np
import pytest

from oracle import work_queue as wq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "paged_kv_attention_persistent_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = "/opt/rocm/bin/hipcc"


def gxx(out, srcs, flags):
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", *flags,
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", out]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    return out


def run(cmd, env=None, timeout=300):
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=timeout)


@pytest.fixture(scope="module")
def fuzz_bin(tmp_path_factory):
    d = tmp_path_factory.mktemp("fuzz")
    return gxx(str(d / "plan_fuzz"), [os.path.join(SAN, "plan_fuzz.cpp"), os.path.join(CSRC, "queue_plan.cpp")],
               ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"])


def test_queue_planner_fuzz_under_asan_ubsan(fuzz_bin):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    for seed in (1, 2, 3):
        r = run([fuzz_bin, "fuzz", str(seed), "3000"], env)
        print(r.stdout.strip())
        assert r.returncode == 0, r.stdout + r.stderr
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
        assert ", 0 failures" in r.stdout


def test_sanitized_planner_queues_equal_the_oracle(fuzz_bin):
    rng = np.random.default_rng(3)
    for trial in range(40):
        B = int(rng.integers(1, 12))
        hkv = int(rng.choice([1, 2, 8]))
        cus = int(rng.choice([8, 64, 256]))
        chunk = int(rng.choice([0, 0, 256, 4096]))
        policy, order = int(rng.integers(0, 3)), int(rng.integers(0, 2))
        lens = rng.integers(0, 40000, size=B)
        lens[rng.random(B) < 0.2] = 0
        r = run([fuzz_bin, "dump", str(hkv), str(cus), str(chunk), str(policy), str(order),
                 *[str(int(x)) for x in lens]])
        assert r.returncode == 0, r.stdout + r.stderr
        head, *rows = r.stdout.strip().splitlines()
        ref = wq.build_queue(lens.tolist(), hkv, cus, chunk, policy, order)
        assert head == f"split {int(ref['split'])} chunk {ref['chunk_tokens']} items {len(ref['items'])}"
        got = np.array([[int(x) for x in row.split()] for row in rows], dtype=np.int64).reshape(-1, 5)
        want = np.stack([ref["items"][f].astype(np.int64) for f in ("seq", "kv_head", "chunk", "tok_begin",
                                                                   "tok_end")], axis=1)
        assert np.array_equal(got, want), f"trial {trial}"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_library_under_asan_ubsan_passes_the_abi_tests(tmp_path):
    lib = str(tmp_path / "libpkv.so")
    srcs = [os.path.join(CSRC, s) for s in ("pkv_kernels.hip", "pkv_api.cpp", "queue_plan.cpp", "pkv_noalloc.hip")]
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-fvisibility=hidden", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan", "-I", os.path.join(ROOT, "include"), *srcs,
           "-o", lib, "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx"]
    r = run(cmd)
    assert r.returncode == 0, r.stderr
    out = run(["nm", "-D", lib]).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out          # instrumented
    rt = run([HIPCC, "--print-file-name=libclang_rt.asan-x86_64.so"]).stdout.strip()
    if not os.path.isabs(rt) or not os.path.exists(rt):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so")
        assert hits, "clang's ASan runtime not found"
        rt = hits[0]
    env = dict(os.environ, LD_PRELOAD=rt, PKV_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", os.path.join(ROOT, "tests",
                                                                                        "test_abi_host.py")],
            env, timeout=600)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[-4000:]


@pytest.fixture(scope="module")
def loop_bins(tmp_path_factory):
    d = tmp_path_factory.mktemp("loop")
    src = [os.path.join(SAN, "loop_protocol.cpp")]
    return (gxx(str(d / "loop_tsan"), src, ["-fsanitize=thread", "-pthread"]),
            gxx(str(d / "loop_plain"), src, ["-pthread"]))


def test_resident_loop_protocol_under_tsan(loop_bins):
    tsan, _ = loop_bins
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66")
    for seed, wgs in ((1, 6), (2, 3), (3, 8)):
        r = run([tsan, "2000", str(wgs), str(seed)], env)
        print(r.stdout.strip())
        assert r.returncode == 0, r.stdout + r.stderr[-4000:]
        assert "ThreadSanitizer" not in r.stderr, r.stderr[-4000:]


def test_loop_protocol_model_catches_an_early_slot_rearm(loop_bins):
    tsan, plain = loop_bins
    for seed in (1, 2, 3):
        r = run([plain, "400", "6", str(seed), "early_rearm"], timeout=120)
        assert r.returncode == 1 and "protocol failure" in r.stderr, (r.returncode, r.stderr[-2000:])
    r = run([tsan, "400", "6", "1", "early_rearm"], dict(os.environ, TSAN_OPTIONS="halt_on_error=1 exitcode=66"),
            timeout=120)
    assert r.returncode in (1, 66), r.returncode
