"""The largest workload, Poisson 13000 x 13000 (169M unknowns, 845M stored
slots, int64 row pointers), 500 fixed CG iterations in the launch
configuration the benchmark times, against the oracle's CG on all of the
process's host threads: x element-wise, the iteration count and the alpha /
beta / r.r history, plus the size-independent properties of the iterate
(energy identity, true vs recursive residual, bit-exact SpMV, Ritz values
inside the closed-form spectrum).  Source of the size: the torch-sla
explainer, Experimental results (2D Poisson up to 169M DOF on one GPU).

It needs about 21 GB of GPU memory and 25 GB of host memory and runs several
minutes on the host (the oracle prints its progress), so it sits in a file
that runs after the other GPU tests."""
import numpy as np
import pytest

import oracle
from test_gpu_fullsize import fixed_vs_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _threads():
    oracle.set_threads(oracle.host_threads())


@pytest.mark.timeout(1200)
def test_poisson13000_int64_fixed500_vs_oracle(capfd):
    fixed_vs_oracle(13000, np.int64, capfd)
