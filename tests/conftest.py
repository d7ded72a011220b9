import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# Collection order: the method's chain first (quantize, GEMM, the full-size
# workloads), then the widened rows, so that under -x a failure in a widened
# row cannot hide the chain's own tests.  Files not listed keep their place
# after these; test_zz_* files stay last.
_ORDER = ["test_oracle_", "test_boundary", "test_bench_cli", "test_gpu_quant.py", "test_gpu_quant_large",
          "test_gpu_gemm.py", "test_gpu_dot_model", "test_gpu_workloads.py", "test_gpu_graph",
          "test_gpu_workspace", "test_gpu_determinism", "test_gpu_recipe", "test_gpu_gemm_fp8out", "test_gpu_transpose",
          "test_gpu_wonly", "test_gpu_packed", "test_gpu_ledger", "test_gpu_workloads_next"]


def _rank(item):
    name = os.path.basename(str(item.fspath))
    if name.startswith("test_zz_"):
        return len(_ORDER) + 1
    for i, prefix in enumerate(_ORDER):
        if name.startswith(prefix):
            return i
    return len(_ORDER)


def pytest_collection_modifyitems(session, config, items):
    items.sort(key=_rank)   # stable: keeps the order inside each file


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (minutes)")


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build(force=False)
    return oracle


def pytest_sessionfinish(session, exitstatus):
    """Write every GEMM acceptance check's statistics (max |err|/S, elements
    above 1e-5 S) as JSON lines to the file FP8RT_PARITY_LOG names, if any."""
    path = os.environ.get("FP8RT_PARITY_LOG")
    mod = sys.modules.get("gpu_helpers")
    if not path or mod is None:
        return
    import json

    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        for st in mod.GEMM_STATS:
            f.write(json.dumps(st) + "\n")
