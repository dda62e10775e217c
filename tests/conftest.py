import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running test")
    # Build only what is missing (a fresh checkout); __graft_entry__.build()
    # always rebuilds everything.
    import __graft_entry__ as ge
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        ge._build_synth()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        ge._build_oracle()
    # The HIP library: built when missing; a binary built from other sources
    # than the checked-out ones stops the run (no test may pass on it).
    import invariant_moe_amd as moe
    if not os.path.exists(moe.LIB_PATH):
        from invariant_moe_amd import _build
        _build.build_library()
    try:
        moe.check_build()
    except moe.MoEError as e:
        raise pytest.UsageError(str(e))


def golden_path(name):
    return os.path.join(ROOT, "tests", "golden", name)


def read_golden(name):
    with open(golden_path(name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
