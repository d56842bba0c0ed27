import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    # A CPU-only session ("-m 'not gpu'") on a fresh checkout builds what the
    # CPU tests load (hipcc cross-compiles for gfx950 without a GPU).  GPU
    # sessions never build: they run what was built beforehand and fail
    # loudly if it is missing.
    if (config.option.markexpr or "").replace(" ", "") == "notgpu":
        import importlib.util
        # load the build script by path: importing the package itself needs
        # the library it is about to build
        spec = importlib.util.spec_from_file_location(
            "_gdn_build", os.path.join(ROOT, "gated_deltanet_decode_amd", "_build.py"))
        _build = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(_build)
        if not (os.path.exists(_build.LIBRARY) and os.path.exists(_build.PROBE_LIBRARY)):
            _build.build()
        if not os.path.exists(_build.C_CHECK_BINARY):
            _build.build_c_check()
        import oracle
        if not os.path.exists(oracle.LIBRARY):
            oracle.build()


def pytest_sessionfinish(session, exitstatus):
    """After a GPU session, write the parity records (one JSON object per
    compared quantity) to parity_records.jsonl in the output folder that the
    GPU runs return."""
    import json
    ref = sys.modules.get("ref")
    if ref is None or not ref.RECORDS:
        return
    out = os.path.join(ROOT, "gpurun_out")
    os.makedirs(out, exist_ok=True)
    with open(os.path.join(out, "parity_records.jsonl"), "w") as f:
        for r in ref.RECORDS:
            f.write(json.dumps(r) + "\n")


@pytest.fixture
def workload():
    """Names the workload a test checks, for its parity records."""
    import ref

    def name(n):
        ref.WORKLOAD["name"] = n
    yield name
    ref.WORKLOAD["name"] = None


@pytest.fixture(scope="session")
def orc():
    import oracle
    if not os.path.exists(oracle.LIBRARY):
        oracle.build()
    return oracle.get()
