"""CPU: sanitizer runs of the oracle and of the C-ABI layer, thread-local
error messages of the C ABI, the input generator's determinism and slice
regeneration, and the package failing loudly without its library."""
import ctypes
import os
import shutil
import subprocess
import sys
import threading

import numpy as np

import gdn_inputs as gi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-ffp-contract=off", "-I", os.path.join(ROOT, "oracle"),
                    os.path.join(ROOT, "tests", "c", "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "gdn_oracle.c"), "-o", exe, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ok" in r.stdout


def test_abi_layer_under_asan_ubsan(tmp_path):
    """gdn_api.cpp built for the host with g++ under ASan/UBSan, its kernel
    launchers replaced by recording stubs (tests/c/gdn_api_stubs.cpp), and
    driven through every entry point's checks and launch arguments by
    tests/c/gdn_api_check.c."""
    csrc = os.path.join(ROOT, "gated_deltanet_decode_amd", "csrc")
    cdir = os.path.join(ROOT, "tests", "c")
    san = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all"]
    inc = ["-I", os.path.join(ROOT, "include"), "-I", csrc, "-I", cdir]
    hip = ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]
    objs = []
    for src, cmd in ((os.path.join(csrc, "gdn_api.cpp"), ["g++", "-std=c++17"] + hip),
                     (os.path.join(cdir, "gdn_api_stubs.cpp"), ["g++", "-std=c++17"] + hip),
                     (os.path.join(cdir, "gdn_api_check.c"), ["gcc", "-std=c99", "-Wall",
                                                               "-Werror"])):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        subprocess.run(cmd + san + inc + ["-c", src, "-o", obj], check=True)
        objs.append(obj)
    exe = str(tmp_path / "gdn_api_check")
    subprocess.run(["g++"] + san + objs + ["-o", exe, "-lm"], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "C ABI host check ok" in r.stdout


def test_last_error_is_thread_local():
    import gated_deltanet_decode_amd as g
    results = {}

    def worker(i):
        d = g.Dims(32, 16, 128, 128)
        # thread i provokes a different error, then reads its own message
        if i == 0:
            rc = g.lib.gdn_step(None, 1, *([None] * 7), None)
        elif i == 1:
            rc = g.lib.gdn_step(ctypes.byref(d), 0, *([None] * 7), None)
        else:
            rc = g.lib.gdn_seq(ctypes.byref(d), 1, 0, *([None] * 7), None)
        for _ in range(200):      # give the other threads time to overwrite a shared buffer
            pass
        results[i] = (rc, g.last_error())

    ths = [threading.Thread(target=worker, args=(i,)) for i in range(3)]
    for t in ths:
        t.start()
    for t in ths:
        t.join()
    assert results[0][0] == -1 and "dims" in results[0][1]
    assert results[1][0] == -2 and "B must be" in results[1][1]
    assert results[2][0] == -2 and "T must be" in results[2][1]
    # a successful-looking validation on this thread clears the message
    assert g.lib.gdn_version() > 0


def test_generator_is_deterministic_and_sliceable():
    a = gi.step_inputs(77, 3, 5)
    b = gi.step_inputs(77, 3, 5)
    for n in a:
        assert np.array_equal(a[n], b[n])
    # sequence 2 alone equals row 2 of the batch (batch independence)
    s = gi.step_inputs(77, 3, 1, b0=2)
    for n in a:
        assert np.array_equal(s[n][0], a[n][2])
    # T = 1 sequence layout equals the single-token layout
    t1 = gi.step_inputs(77, 3, 5, T=1)
    for n in a:
        assert np.array_equal(t1[n][:, 0], a[n])
    # another slot or seed gives other numbers
    c = gi.step_inputs(78, 3, 5)
    assert not np.array_equal(c["v"], a["v"])
    M = gi.state(77, 3, 4)
    assert np.array_equal(gi.state(77, 3, 1, b0=3)[0], M[3])
    # distributions: unit-norm q and k, beta in (0,1), gate < 0, state std 0.1
    assert np.allclose(np.linalg.norm(a["q"].astype(np.float64), axis=-1), 1, atol=1e-6)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1)) and np.all(a["gate"] < 0)
    assert abs(float(M.std()) - 0.1) < 0.002


def test_package_fails_loudly_without_its_library(tmp_path):
    pkg = tmp_path / "gated_deltanet_decode_amd"
    pkg.mkdir()
    for fn in ("__init__.py", "_build.py"):
        shutil.copy(os.path.join(ROOT, "gated_deltanet_decode_amd", fn), pkg / fn)
    r = subprocess.run([sys.executable, "-c", "import gated_deltanet_decode_amd"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "ImportError" in r.stderr and "not built" in r.stderr


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with a message before
    touching a GPU."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
