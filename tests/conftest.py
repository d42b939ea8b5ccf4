import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (seconds to minutes)")


def read_golden(name):
    """Parse a golden fixture: '#' comments, then 'key v1 v2 ...' lines."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


@pytest.fixture
def golden():
    return read_golden


LIB = os.path.join(ROOT, "mxfp4_mixture_experts_moe_amd", "libk3moe.so")


@pytest.fixture(scope="session")
def k3():
    """The HIP library's Python binding (built in-tree first if nothing is built)."""
    if not os.path.exists(LIB):
        import importlib.util

        spec = importlib.util.spec_from_file_location("_k3moe_build", os.path.join(ROOT, "mxfp4_mixture_experts_moe_amd", "build.py"))
        builder = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(builder)
        builder.build(verbose=False)
    import mxfp4_mixture_experts_moe_amd as m

    return m


@pytest.fixture(scope="session")
def k3_experts(k3):
    """All 896 K3-shaped experts resident on the device (15.7 GB), shared by
    every GPU test module that needs them."""
    import moe_inputs
    from moe_inputs.device import upload_experts
    from tests.gpu_util import expert_blocks

    print("[k3] uploading 896 K3 experts", flush=True)
    return upload_experts(moe_inputs.PREFILL, expert_blocks(k3))
