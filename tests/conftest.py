import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large workload; runs in a few tens of seconds")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _selections_completed(request):
    """After every GPU test: no selection on a cached workspace of the binding gave up
    (tg_select_check on each; tests with their own workspaces check those themselves)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    binding = sys.modules.get("learned_token_pruning_scorer_amd.binding")
    if binding is None:
        return
    for ws in list(binding._workspaces.values()):
        binding.tg_select_check(ws)
