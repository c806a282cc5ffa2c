import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def _ensure_built():
    """Builds the HIP libraries in-tree only when none is there (a fresh
    checkout); an existing build is used as it is."""
    lib = os.path.join(ROOT, "compressed_sparse_kv_compress_amd", "libcskv.so")
    synth_lib = os.path.join(ROOT, "synth", "libcskv_synth.so")
    if not (os.path.exists(lib) and os.path.exists(synth_lib)):
        import __graft_entry__

        __graft_entry__.build()


def pytest_configure(config):
    _ensure_built()
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size workload checks (still run with -m gpu)")


def pytest_collection_modifyitems(config, items):
    # GPU tests fail loudly without a device rather than skipping silently, but
    # only when GPU tests were asked for; a plain run on a CPU machine deselects them.
    markexpr = config.getoption("-m") or ""
    if "gpu" in markexpr and "not gpu" not in markexpr:
        return
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:
        has_gpu = False
    if not has_gpu:
        skip = pytest.mark.skip(reason="no GPU in this container")
        for item in items:
            if "gpu" in item.keywords:
                item.add_marker(skip)
