import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def full_experts():
    """Expert weights of the full-shape workloads (identical recipe and seed
    for decode, prefill, skewed and long; 9.1 GB), generated once per
    session, host + device."""
    import synth
    from tests import gpu_util as gu
    wl = synth.WORKLOADS["decode"]
    gu.note("  generating full-shape expert weights (9.1 GB)")
    host = synth.gen_experts(wl)
    dev = tuple(gu.to_dev(a) for a in host)
    return host, dev


@pytest.hookimpl(trylast=True)
def pytest_runtest_logfinish(nodeid, location):
    """Flush the progress line after every test, so that a long GPU session
    shows each test's end as it happens (stdout to a file or pipe is block
    buffered)."""
    tr = _CONFIG[0].pluginmanager.get_plugin("terminalreporter") if _CONFIG else None
    if tr is not None:
        tr._tw.flush()


_CONFIG = []


@pytest.hookimpl(tryfirst=True)
def pytest_sessionstart(session):
    _CONFIG.append(session.config)
    # a fresh checkout has no libmoe.so: compile it once (the oracle and the
    # input generator compile themselves on first use)
    from sparse_moe_layer_fp32_amd import _build
    _build.ensure_built()
