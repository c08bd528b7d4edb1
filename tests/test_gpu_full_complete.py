"""Complete parity at the benchmark's full workload shapes (configs 2-5), through
np_decode_step as bench.py calls it (a compute and a copy stream), with the row
store both in HBM and in pinned host memory (the placement the workloads specify: the delta
bundles cross the host link every token). See tests/full_run.py for what is compared:
state at every (step, layer), every layer's whole buffer at steps 0, 1, T/2 and T-1, y at
every (step, layer), and a back-to-back replay without synchronization.

Config 5 (47 layers of 1.23 GB row stores, 58 GB in all) runs in three groups of layers, each
from its own cold start: its pinned stores do not all fit the host's pinned-memory limit at
once. The layers of a decode step are independent in their state, so a group's run is the
full run restricted to those layers.
"""
import pytest

from tests.full_run import run_complete

pytestmark = pytest.mark.gpu


@pytest.mark.timeout(600)
@pytest.mark.parametrize("num", [2, 3, 4])
def test_complete_parity(num):
    run_complete(num)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("group", [range(0, 16), range(16, 32), range(32, 47)], ids=["l0-15", "l16-31", "l32-46"])
def test_complete_parity_config5(group):
    run_complete(5, list(group))
